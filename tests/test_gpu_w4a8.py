"""GPU parity of the W4A8 path: per-token FP8 (E4M3) activation
quantization (bit-exact codes and scales against the oracle, both layouts),
its dequantization, and the W4A8 GEMM (INT4 g128 weights x FP8 activations
on FP8 matrix cores) against the oracle's fp64 product within the tolerance
of q4_helpers, plus exact special cases."""
import numpy as np
import pytest
import torch

import oracle
import w4_gemm_amd as q4
from w4_gemm_amd import workloads
from q4_helpers import check_matmul, log, to_f32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def fp8_untile(codes: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Tiled FP8 layout (include/q4.h) -> row-major [rows, cols]: tile (t, s)
    of 2048 bytes; operand byte 4d + i of lane l = 16g + n (d = 2w + h) holds
    k = 128s + 32g + 8w + 2i + h of row 16t + n; operand bytes 0..15 of lane
    l at 16l, bytes 16..31 at 1024 + 16l."""
    RT, S = (rows + 15) // 16, cols // 128
    c = codes.reshape(RT, S, 2, 4, 16, 16)        # t, s, half, g, n, byte-in-half
    out = np.zeros((RT * 16, cols), dtype=np.uint8)
    for half in range(2):
        for b in range(16):
            p = 16 * half + b                      # operand byte
            d, i = p // 4, p % 4
            w, h = d // 2, d % 2
            for g in range(4):
                k = np.arange(S) * 128 + 32 * g + 8 * w + 2 * i + h
                out[:, k] = c[:, :, half, g, :, b].transpose(0, 2, 1).reshape(RT * 16, S)
    return out[:rows], out[rows:]


def fp8_inputs(rows, cols, seed):
    a = workloads.matrix(f"t8/a{rows}x{cols}", rows, cols, 1.0, seed=seed,
                         channel_frac=0.01, channel_mult=10.0)
    a = a.clone()
    if rows > 2:
        a[1] = 0.0                                 # an all-zero row
        a[2, :5] = -0.0
    return a


@pytest.mark.parametrize("layout", ("rows", "tiled"))
@pytest.mark.parametrize("rows,cols", [(1, 512), (5, 1024), (17, 512), (130, 2048), (64, 4096),
                                       (3, 96), (40, 208), (7, 8192), (3, 8704), (2, 16384),
                                       (2050, 1024), (2048, 8192)])
def test_fp8_rows_quantize_bit_exact(rows, cols, layout):
    """Rows up to 8192 values are quantized by a workgroup holding the row
    in registers; longer ones (8704, 16384) by a wave reading it twice;
    2050 rows end in a ragged tile."""
    if layout == "tiled" and cols % 512:
        pytest.skip("the tiled layout needs cols % 512 == 0")
    log("fp8 quantize", layout, rows, cols)
    a = fp8_inputs(rows, cols, seed=61)
    qg = q4.quantize(a.to(DEV), "fp8_row", layout=layout)
    torch.cuda.synchronize()
    qr = oracle.quantize_fp8_rows(to_f32(a))
    codes = qg.codes.cpu().numpy()
    if layout == "tiled":
        codes, pad = fp8_untile(codes, rows, cols)
        assert not pad.any()
    bad = np.argwhere(codes != qr.codes)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()}"
    assert np.array_equal(qg.scales.cpu().numpy(), qr.scales)
    # dequantization (fp32 and bf16) against the oracle's
    ref = oracle.dequant_fp8_rows(qr)
    d32 = torch.empty((rows, cols), dtype=torch.float32, device=DEV)
    q4.q4_dequant(qg, d32)
    d16 = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    q4.q4_dequant(qg, d16)
    torch.cuda.synchronize()
    assert np.array_equal(d32.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    exp16 = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(ref))
    assert np.array_equal(d16.cpu().float().numpy().view(np.uint32), exp16.view(np.uint32))


def _fp8_quantize_matches_oracle(a: torch.Tensor, layout="rows"):
    rows, cols = a.shape
    qg = q4.quantize(a.to(DEV), "fp8_row", layout=layout)
    torch.cuda.synchronize()
    qr = oracle.quantize_fp8_rows(to_f32(a))
    codes = qg.codes.cpu().numpy()
    if layout == "tiled":
        codes, _ = fp8_untile(codes, rows, cols)
    bad = np.argwhere(codes != qr.codes)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()}"
    assert np.array_equal(qg.scales.cpu().numpy(), qr.scales)


@pytest.mark.parametrize("width", (512, 1024, 4096))
def test_fp8_rows_quantize_all_bf16_values(width):
    """Every finite bf16 value, sorted by magnitude into rows of `width` (1,
    2 and 8 octaves below each row's largest value, so the quotients cover
    the normal E4M3 codes and, for the widest rows, the subnormal ones), with
    random signs, in random order within each row."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = np.sort(np.abs(v[np.isfinite(v)]))[::-1]
    n = (v.size // width) * width
    rng = np.random.default_rng(81)
    x = (v[:n] * np.where(rng.random(n) < 0.5, -1, 1)).reshape(-1, width).astype(np.float32)
    x = rng.permuted(x, axis=1)
    log("fp8 all bf16", x.shape)
    for layout in ("rows", "tiled"):
        _fp8_quantize_matches_oracle(torch.from_numpy(x).to(torch.bfloat16), layout)


def test_fp8_rows_quantize_exact_ties():
    """Rows whose largest magnitude is 448 2^e have scale 2^e exactly; their
    other values are the midpoints between consecutive E4M3 values (the
    subnormal ones (2k+1) 2^-10 and the normal ones up to 448) times 2^e, of
    both signs: ties, which go to the even code."""
    e4m3 = np.array([oracle.e4m3_value(c) for c in range(0x7F)], np.float64)  # 0 .. 448
    mids = ((e4m3[:-1] + e4m3[1:]) / 2).astype(np.float32)
    rows = []
    for e in range(-8, 8):
        row = np.zeros(512, np.float32)
        row[0] = 448.0 * 2.0 ** e
        row[1:1 + mids.size] = mids * 2.0 ** e
        row[1 + mids.size:1 + 2 * mids.size] = -mids * 2.0 ** e
        rows.append(row)
    x = np.stack(rows)
    a = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(to_f32(a), x)  # every midpoint is exact in bf16
    for layout in ("rows", "tiled"):
        _fp8_quantize_matches_oracle(a, layout)


def _w4a8_case(M, N, K, alayout, wlayout, seed):
    w = workloads.matrix(f"t8/w{N}x{K}", N, K, 0.02, seed=seed)
    a = fp8_inputs(M, K, seed + 1)
    qw = q4.quantize(w.to(DEV), "int4", layout=wlayout)
    qa = q4.quantize(a.to(DEV), "fp8_row", layout=alayout)
    return a, w, qa, qw


@pytest.mark.parametrize("alayout,wlayout", [("tiled", "tiled"), ("rows", "rows"),
                                             ("rows", "tiled"), ("tiled", "rows")])
@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (100, 300, 1024), (1, 16, 512), (300, 520, 1536),
                                   (16, 1000, 2048), (33, 64, 256)])
def test_gemm_w4a8_small(M, N, K, alayout, wlayout):
    if "tiled" in (alayout, wlayout) and K % 512:
        pytest.skip("the tiled layout needs K % 512 == 0")
    log("gemm w4a8", alayout, wlayout, M, N, K)
    a, w, qa, qw = _w4a8_case(M, N, K, alayout, wlayout, seed=71)
    C = torch.full((M, N + 4), float("nan"), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(qa, qw, C[:, :N])
    torch.cuda.synchronize()
    Cc = C.cpu()
    assert torch.isnan(Cc[:, N:]).all()
    qwr = oracle.quantize("int4", to_f32(w))
    qar = oracle.quantize_fp8_rows(to_f32(a))
    ad, wd = oracle.dequant_fp8_rows(qar), oracle.dequant(qwr)
    e = check_matmul(Cc[:, :N], oracle.gemm_w4a8(None, qwr, aq=qar), ad, wd, True, "w4a8")
    log("w4a8 max normalized error", e)


@pytest.mark.parametrize("layout", ("rows", "tiled"))
def test_w4a8_one_hot_rows_return_weight_columns(layout):
    """A row holding 448 at column c and zeros elsewhere has scale exactly 1
    and code 0x7E, so the output row is bf16(448 * w'[:, c]) exactly."""
    N, K = 272, 1024
    w = workloads.matrix("t8/oh", N, K, 0.05, seed=73)
    cols = np.array([0, 1, 127, 128, 511, 512, 700, 1023])
    a = torch.zeros((len(cols), K), dtype=torch.bfloat16)
    a[torch.arange(len(cols)), torch.from_numpy(cols)] = 448.0
    qw = q4.quantize(w.to(DEV), "int4", layout=layout)
    qa = q4.quantize(a.to(DEV), "fp8_row", layout=layout)
    C = torch.empty((len(cols), N), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(qa, qw, C)
    torch.cuda.synchronize()
    wd = oracle.dequant(oracle.quantize("int4", to_f32(w)))
    exp = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits((448.0 * wd[:, cols].T).astype(np.float32)))
    assert np.array_equal(C.cpu().float().numpy(), exp)


def test_w4a8_deterministic():
    a, w, qa, qw = _w4a8_case(300, 520, 1536, "tiled", "tiled", seed=75)
    outs = []
    for _ in range(3):
        C = torch.empty((300, 520), dtype=torch.bfloat16, device=DEV)
        q4.q4_gemm(qa, qw, C)
        outs.append(C)
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_full_w4a8_prefill_gemm():
    """4096x8192x8192 W4A8 in the benchmark's layouts; 64 sampled rows of C."""
    wl = workloads.w4a8_gemm()
    A, W = wl.tensors["A"], wl.tensors["W"]
    M, N = A.shape[0], W.shape[0]
    log("w4a8: quantize (tiled, the benchmark's layout)")
    qw = q4.quantize(W.to(DEV), "int4", layout="tiled")
    qa = q4.quantize(A.to(DEV), "fp8_row", layout="tiled")
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(qa, qw, C)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(76).choice(M, 62, replace=False)]))
    qwr = oracle.quantize("int4", to_f32(W))
    qar = oracle.quantize_fp8_rows(to_f32(A[torch.from_numpy(rows)]))
    ad, wd = oracle.dequant_fp8_rows(qar), oracle.dequant(qwr)
    e = check_matmul(C.cpu()[torch.from_numpy(rows)], oracle.gemm_w4a8(None, qwr, aq=qar), ad, wd,
                     True, "w4a8 prefill")
    log("w4a8 prefill max normalized error", e)
