"""GPU parity of q4_gemm_quantized, the GEMM whose epilogue writes C already
quantized (MXFP4, or NVFP4 under a given tensor scale) for the next W4A4
layer ("Quantization in deployment", Exercises, "The cost of block FP8":
activation scales computed at the end of the previous kernel).

The reference is the unfused path on the same inputs: q4_gemm's bf16 C,
quantized by the oracle (and, for the whole tiled buffer with its padding
rows, by q4_quantize).  Codes, scales and the NVFP4 tensor scale must agree
bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import w4_gemm_amd as q4
from w4_gemm_amd import workloads
from q4_helpers import assert_quant_equal, log, scales_np, to_f32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gs_tensor(v):
    return torch.tensor([v], dtype=torch.float32, device=DEV)


def _nv_scales(c_f32):
    """Tensor scales to quantize C with: the one of C's own amax (a
    calibrated scale), a quarter of it (block scales clamp at 448 and
    values saturate at 6) and 300 times it (small blocks' E4M3 scales
    underflow to 0)."""
    amax = float(np.abs(c_f32).max())
    g = np.float32(np.float32(max(amax, 1e-12)) / np.float32(2688.0))
    return [float(g), float(np.float32(g * np.float32(0.25))), float(np.float32(g * np.float32(300.0)))]


def _check(cq, c_bf16, ofmt, gs=None):
    """cq (fused) against the oracle's quantization of the unfused bf16 C, and
    in the tiled layout against q4_quantize's whole buffer (padding too)."""
    c32 = to_f32(c_bf16)
    ref = oracle.quantize(ofmt, c32, gs=gs)
    assert_quant_equal(cq, ref, ofmt)
    if cq.layout == q4.LAYOUT_TILED:
        qg = q4.quantize(c_bf16, ofmt, None if gs is None else _gs_tensor(gs), layout="tiled")
        torch.cuda.synchronize()
        assert torch.equal(qg.codes, cq.codes), "tiled code bytes (padding rows included)"
        assert np.array_equal(scales_np(qg, ofmt), scales_np(cq, ofmt))


def _fused(A, W, ofmt, olayout, M, N, gs=None):
    cq = q4.empty_q4(ofmt, M, N, device=DEV, layout=olayout)
    # sentinels: every byte the call should write is overwritten
    cq.codes.fill_(0xA5)
    cq.scales.fill_(0x5A)
    if cq.global_scale is not None:
        cq.global_scale.fill_(-1.0)
    q4.q4_gemm_quantized(A, W, cq, None if gs is None else _gs_tensor(gs))
    torch.cuda.synchronize()
    return cq


@pytest.mark.parametrize("olayout", ["rows", "tiled"])
@pytest.mark.parametrize("ofmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("wfmt", ["int4", "mxfp4", "nvfp4", "int4_zp"])
def test_w4a16_quantized_output(wfmt, ofmt, olayout):
    M, N, K = 300, 1024, 1024          # 2 x 4 blocks of 256 x 256, a ragged row tail (300 % 16 = 12)
    log("w4a16 fused quantize", wfmt, ofmt, olayout, M, N, K)
    w = workloads.matrix("fq/w", N, K, 0.02, seed=71, outlier_frac=0.001, outlier_mult=20.0)
    a = workloads.matrix("fq/a", M, K, 1.0, seed=72).to(DEV)
    W = q4.quantize(w.to(DEV), wfmt, layout="tiled")
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(a, W, C)
    torch.cuda.synchronize()
    for gs in (_nv_scales(to_f32(C)) if ofmt == "nvfp4" else [None]):
        cq = _fused(a, W, ofmt, olayout, M, N, gs)
        _check(cq, C, ofmt, gs)


@pytest.mark.parametrize("ofmt", ["mxfp4", "nvfp4"])
def test_w4a16_quantized_output_ragged_columns(ofmt):
    """N = 544: the last 256-column block holds one 32-column block (row-major
    output; the tiled layout needs N % 512 == 0)."""
    M, N, K = 40, 544, 512
    w = workloads.matrix("fq/w2", N, K, 0.02, seed=73)
    a = workloads.matrix("fq/a2", M, K, 1.0, seed=74).to(DEV)
    W = q4.quantize(w.to(DEV), "mxfp4", layout="tiled")
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(a, W, C)
    torch.cuda.synchronize()
    gs = _nv_scales(to_f32(C))[0] if ofmt == "nvfp4" else None
    _check(_fused(a, W, ofmt, "rows", M, N, gs), C, ofmt, gs)


@pytest.mark.parametrize("olayout", ["rows", "tiled"])
@pytest.mark.parametrize("ofmt", ["mxfp4", "nvfp4"])
def test_w4a4_quantized_output(ofmt, olayout):
    M, N, K = 300, 1024, 1024
    log("w4a4 fused quantize", ofmt, olayout, M, N, K)
    w = workloads.matrix("fq/w4", N, K, 0.02, seed=75)
    a = workloads.matrix("fq/a4", M, K, 1.0, seed=76).to(DEV)
    W = q4.quantize(w.to(DEV), "mxfp4", layout="tiled")
    Aq = q4.quantize(a, "mxfp4", layout="tiled")
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(Aq, W, C)
    torch.cuda.synchronize()
    for gs in (_nv_scales(to_f32(C)) if ofmt == "nvfp4" else [None]):
        _check(_fused(Aq, W, ofmt, olayout, M, N, gs), C, ofmt, gs)


def test_w4a4_chain_full_size():
    """The W4A4 workload (8192^3) as one layer of a chain: its output
    quantized to MXFP4 (tiled) by the epilogue is byte for byte what
    q4_quantize makes of the bf16 output, and sampled rows match the oracle;
    the quantized output then feeds the next W4A4 GEMM directly."""
    M = N = K = 8192
    log("w4a4 chain full size", M, N, K)
    a = workloads.matrix("fq/aF", M, K, 1.0, seed=77).to(DEV)
    w = workloads.matrix("fq/wF", N, K, 0.02, seed=78).to(DEV)
    Aq = q4.quantize(a, "mxfp4", layout="tiled")
    W = q4.quantize(w, "mxfp4", layout="tiled")
    del a, w
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(Aq, W, C)
    cq = _fused(Aq, W, "mxfp4", "tiled", M, N)
    qg = q4.quantize(C, "mxfp4", layout="tiled")
    torch.cuda.synchronize()
    assert torch.equal(qg.codes, cq.codes) and torch.equal(qg.scales, cq.scales)
    rows = np.random.default_rng(79).choice(M, 48, replace=False)
    c_rows = to_f32(C[torch.from_numpy(rows).to(DEV)])
    ref = oracle.quantize("mxfp4", c_rows)
    assert_quant_equal(cq, ref, "mxfp4", rows=rows)
    # the next layer consumes the fused output as its A operand
    C2 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    C3 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(cq, W, C2)
    q4.q4_gemm(qg, W, C3)
    torch.cuda.synchronize()
    assert torch.equal(C2, C3)

