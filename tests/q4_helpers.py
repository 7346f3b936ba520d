"""Shared helpers of the GPU parity tests: moving tensors, running the
oracle on the same inputs, and the matmul tolerance.

Matmul tolerance (per output element, in the test, both must hold):
  * gate:  |C - ref| <= 2e-2 * ||a_m||_2 * ||w'_n||_2
  * tight: |C - ref| <= 2^-8 |ref| + c * sum_k |a_mk| |w'_nk|
    with c = 2^-16 when every product a*w' is exact in the kernel (bf16 x
    and MXFP4 weights, or MXFP4 x MXFP4), and c = 2^-8 when the kernel
    rounds w' to bf16 once (INT4, NVFP4: at most 2^-9 relative per
    product).  2^-8 |ref| covers the bf16 output rounding (2^-9) with room
    for the fp32 accumulation.
"""
import sys

import numpy as np
import torch

import oracle

FMT_ID = {"int4": 0, "mxfp4": 1, "nvfp4": 2, "int4_zp": 4}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def scales_np(q, fmt):
    s = q.scales.cpu()
    if fmt == "int4":
        return s.view(torch.int16).numpy().view(np.uint16)
    if fmt == "int4_zp":
        return s.view(torch.int32).numpy().view(np.uint32)
    return s.numpy()


def untile(codes: np.ndarray, scales: np.ndarray, fmt: str, rows: int, cols: int):
    """Tiled layout -> row-major (codes [rows, cols/2], scales [rows, cols/g]),
    following the tiled layout's definition in include/q4.h: tile (t, s) of
    1 KB holds, at bytes [16l, 16l+16) with l = 16g + n, the codes of row
    16t+n, k = 128s + 32g .. +32; scales are grouped by four super-chunks."""
    RT, S = (rows + 15) // 16, cols // 128
    Q = S // 4
    c = codes.reshape(RT, S, 4, 16, 16)                 # t, s, g, n, byte
    c = c.transpose(0, 3, 1, 2, 4).reshape(RT * 16, S * 64)[:rows]
    if fmt == "mxfp4":
        sc = scales.reshape(RT, Q, 4, 16, 4)            # t, q, g, n, i
        sc = sc.transpose(0, 3, 1, 4, 2).reshape(RT * 16, Q * 16)
    elif fmt == "nvfp4":
        sc = scales.reshape(RT, Q, 4, 16, 4, 2)         # t, q, g, n, i, h
        sc = sc.transpose(0, 3, 1, 4, 2, 5).reshape(RT * 16, Q * 32)
    else:
        sc = scales.reshape(RT, Q, 16, 4)               # t, q, n, i
        sc = sc.transpose(0, 2, 1, 3).reshape(RT * 16, Q * 4)
    return np.ascontiguousarray(c), np.ascontiguousarray(sc[:rows])


def assert_quant_equal(q_gpu, q_ref, fmt, rows=None):
    codes = q_gpu.codes.cpu().numpy()
    sc = scales_np(q_gpu, fmt)
    if q_gpu.layout == 1:
        codes, sc = untile(codes, sc, fmt, q_gpu.rows, q_gpu.cols)
    if rows is not None:
        codes, sc = codes[rows], sc[rows]
    assert codes.shape == q_ref.codes.shape
    bad = np.argwhere(codes != q_ref.codes)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first {bad[:5].tolist()}"
    bad = np.argwhere(sc != q_ref.scales)
    assert bad.size == 0, f"{len(bad)} scales differ, first {bad[:5].tolist()}"
    if fmt == "nvfp4":
        assert q_gpu.global_scale.item() == np.float32(q_ref.gs), (q_gpu.global_scale.item(), q_ref.gs)


def check_matmul(got: torch.Tensor, ref: np.ndarray, a: np.ndarray, wd: np.ndarray,
                 exact_products: bool, what: str = ""):
    """got: bf16 output (any device); ref: fp64; a [M,K] and wd [N,K] the
    operands as the oracle used them.  Returns the max error normalized by
    ||a_m|| ||w'_n||."""
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    a64 = a.astype(np.float64)
    w64 = wd.astype(np.float64)
    err = np.abs(g - ref)
    scale = np.outer(np.linalg.norm(a64, axis=1), np.linalg.norm(w64, axis=1))
    gate = 2e-2 * scale
    c = 2.0 ** -16 if exact_products else 2.0 ** -8
    tight = 2.0 ** -8 * np.abs(ref) + c * (np.abs(a64) @ np.abs(w64).T) + 1e-30
    bad = np.argwhere(err > gate)
    assert bad.size == 0, f"{what}: {len(bad)} elements beyond the 2e-2 gate, first {bad[:3].tolist()}"
    bad = np.argwhere(err > tight)
    assert bad.size == 0, (f"{what}: {len(bad)} elements beyond the derived bound, first "
                           f"{[(int(i), int(j), g[i, j], ref[i, j]) for i, j in bad[:3]]}")
    with np.errstate(invalid="ignore", divide="ignore"):
        nerr = np.where(scale > 0, err / scale, 0.0)
    return float(nerr.max()) if nerr.size else 0.0
