"""GPU parity of the W4 matmuls (q4_gemv, q4_gemm W4A16 / W4A4,
q4_grouped_gemm) against the oracle's fp64 references, within the
tolerance stated in q4_helpers (gate 2e-2 ||a|| ||w'|| plus a derived
per-element bound), plus special cases with exact answers, unwritten-output
sentinels and run-to-run determinism."""
import numpy as np
import pytest
import torch

import oracle
import w4_gemm_amd as q4
from w4_gemm_amd import workloads
from q4_helpers import check_matmul, log, to_f32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FMTS = ("int4", "mxfp4", "nvfp4", "int4_zp")
EXACT = {"int4": False, "mxfp4": True, "nvfp4": False, "int4_zp": False}


def quantized(w_bf16, fmt, layout="rows"):
    qg = q4.quantize(w_bf16.to(DEV), fmt, layout=layout)
    qr = oracle.quantize(fmt, to_f32(w_bf16))
    return qg, qr


def tiled_ok(K, rows=16):
    return K % 512 == 0 and rows % 16 == 0


LAYOUTS = ("rows", "tiled")


# --------------------------------------------------------------------------
# GEMV
# --------------------------------------------------------------------------
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(1000, 1024), (77, 384), (4100, 1280), (16400, 2048), (40, 512)])
def test_gemv_small(fmt, N, K, layout):
    if layout == "tiled" and not tiled_ok(K):
        pytest.skip("the tiled layout needs K % 512 == 0")
    log("gemv", fmt, layout, N, K)
    w = workloads.matrix(f"tg/w{N}x{K}", N, K, 0.02, seed=21, outlier_frac=0.001, outlier_mult=20.0)
    qg, qr = quantized(w, fmt, layout)
    wd = oracle.dequant(qr)
    for B in (1, 3, 9, 16):
        x = workloads.matrix(f"tg/x{B}x{K}", B, K, 1.0, seed=22)
        y = torch.full((B, N + 8), float("nan"), dtype=torch.bfloat16, device=DEV)
        q4.q4_gemv(qg, x.to(DEV), y[:, :N])
        torch.cuda.synchronize()
        yc = y.cpu()
        assert torch.isnan(yc[:, N:]).all()       # nothing written past N
        ref = oracle.matmul_f64(to_f32(x), wd)
        check_matmul(yc[:, :N], ref, to_f32(x), wd, EXACT[fmt], f"gemv {fmt} B={B}")


def tiny_rows(N, K, seed):
    """Weights whose rows span many magnitudes (row n scaled by 10^-(n % 6)):
    INT4 groups of the small rows get fp16-subnormal scales, NVFP4 blocks
    E4M3-subnormal scales, MXFP4 blocks small E8M0 exponents."""
    w = workloads.matrix(f"tg/tiny{N}x{K}", N, K, 0.02, seed=seed).float()
    w *= torch.tensor([10.0 ** -(n % 6) for n in range(N)]).reshape(N, 1)
    return w.to(torch.bfloat16)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_tiny_scales(fmt, layout):
    N, K = 96, 1024
    w = tiny_rows(N, K, 28)
    qg, qr = quantized(w, fmt, layout)
    wd = oracle.dequant(qr)
    sc = np.asarray(qr.scales).astype(np.int64).ravel()   # the case is really there
    if fmt in ("int4", "int4_zp"):
        assert np.any(((sc & 0x7C00) == 0) & ((sc & 0x3FF) != 0))    # fp16 subnormal
    elif fmt == "nvfp4":
        assert np.any(((sc & 0x78) == 0) & ((sc & 0x7) != 0))        # E4M3 subnormal
    for B in (1, 16):
        x = workloads.matrix(f"tg/tinyx{B}", B, K, 1.0, seed=29)
        y = torch.empty((B, N), dtype=torch.bfloat16, device=DEV)
        q4.q4_gemv(qg, x.to(DEV), y)
        torch.cuda.synchronize()
        check_matmul(y.cpu(), oracle.matmul_f64(to_f32(x), wd), to_f32(x), wd, EXACT[fmt],
                     f"gemv tiny {fmt} B={B}")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_one_hot_x_returns_a_column(fmt, layout):
    N, K = 300, 512
    w = workloads.matrix("tg/onehot", N, K, 0.05, seed=23)
    qg, qr = quantized(w, fmt, layout)
    wd = oracle.dequant(qr)
    for k in (0, 129, 511):
        x = torch.zeros((1, K), dtype=torch.bfloat16)
        x[0, k] = 1.0
        y = torch.empty((1, N), dtype=torch.bfloat16, device=DEV)
        q4.q4_gemv(qg, x.to(DEV), y)
        torch.cuda.synchronize()
        got = y.cpu().float().numpy()[0]
        # x is one-hot, so the sum is the single product x_k * w'_nk, rounded
        # once to bf16 (values compared, so a sum of +0 and -0 may give +0)
        exp = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(wd[:, k]))
        assert np.array_equal(got, exp)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gemv_all_ones_accumulates_in_fp32(layout):
    """All-ones weights and x over K = 1024 must give exactly 1024; a bf16
    accumulator would stop at 256."""
    K = 1024
    w = torch.ones((64, K), dtype=torch.bfloat16)
    qg, _ = quantized(w, "mxfp4", layout)
    y = torch.empty((1, 64), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemv(qg, torch.ones((1, K), dtype=torch.bfloat16, device=DEV), y)
    torch.cuda.synchronize()
    assert torch.all(y.cpu().float() == 1024.0)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gemv_batch_rows_are_independent(layout):
    """Row b of a B=16 GEMV equals the B=1 GEMV of that row, bit for bit."""
    N, K = 2048, 2048
    w = workloads.matrix("tg/batch", N, K, 0.02, seed=24)
    qg, _ = quantized(w, "mxfp4", layout)
    x = workloads.matrix("tg/batchx", 16, K, 1.0, seed=25).to(DEV)
    y16 = torch.empty((16, N), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemv(qg, x, y16)
    for b in (0, 5, 15):
        y1 = torch.empty((1, N), dtype=torch.bfloat16, device=DEV)
        q4.q4_gemv(qg, x[b:b + 1], y1)
        torch.cuda.synchronize()
        assert torch.equal(y1[0], y16[b])


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gemv_deterministic(layout):
    N, K = 4096, 4096
    w = workloads.matrix("tg/det", N, K, 0.02, seed=26)
    qg, _ = quantized(w, "mxfp4", layout)
    x = workloads.matrix("tg/detx", 4, K, 1.0, seed=27).to(DEV)
    a = torch.empty((4, N), dtype=torch.bfloat16, device=DEV)
    b = torch.empty((4, N), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemv(qg, x, a)
    q4.q4_gemv(qg, x, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_row_major_scales_at_any_alignment(fmt):
    """The row-major GEMV loads a step's row scales in vector loads when K %
    512 == 0 and the scale rows are aligned to the vector, and one scale per
    super-chunk otherwise: the same tensor with its scales 4 bytes off that
    alignment gives the same bytes."""
    N, K = 300, 2048
    w = workloads.matrix("tg/salign", N, K, 0.02, seed=31)
    qg, _ = quantized(w, fmt, "rows")
    x = workloads.matrix("tg/salignx", 16, K, 1.0, seed=32).to(DEV)
    nb = qg.scales.numel() * qg.scales.element_size()
    buf = torch.empty(nb + 64, dtype=torch.uint8, device=DEV)
    base = (-buf.data_ptr()) % 16                       # 16-byte aligned start inside buf
    off = buf[base + 4: base + 4 + nb]                  # 4-byte aligned, not 8- or 16-byte
    off.copy_(qg.scales.reshape(-1).view(torch.uint8))
    qo = q4.Q4Tensor(qg.fmt, N, K, qg.codes, off.view(qg.scales.dtype).reshape(qg.scales.shape),
                     qg.global_scale, qg.layout)
    assert qo.scales.data_ptr() % 16 == 4
    a = torch.empty((16, N), dtype=torch.bfloat16, device=DEV)
    b = torch.empty_like(a)
    q4.q4_gemv(qg, x, a)
    q4.q4_gemv(qo, x, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_full_int4_gemv(layout):
    wl = workloads.int4_gemv()
    qg, qr = quantized(wl.tensors["W"], "int4", layout)
    x = wl.tensors["x"]
    y = torch.empty((1, 1024), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemv(qg, x.to(DEV), y)
    torch.cuda.synchronize()
    wd = oracle.dequant(qr)
    e = check_matmul(y.cpu(), oracle.matmul_f64(to_f32(x), wd), to_f32(x), wd, False, "int4 1024")
    log("int4 g128 gemv max normalized error", e)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_full_mxfp4_decode_gemv(layout):
    """28672 x 8192 MXFP4, B = 1, 4, 16: 512 sampled output columns n (all
    batch rows) against the oracle; the tiled case is the benchmark's."""
    wl = workloads.mxfp4_gemv()
    W = wl.tensors["W"]
    N, K = W.shape
    log("mxfp4 decode gemv: quantize", layout)
    qg = q4.quantize(W.to(DEV), "mxfp4", layout=layout)
    rows = np.sort(np.random.default_rng(28).choice(N, 512, replace=False))
    rows[:3] = [0, N // 2, N - 1]
    rows = np.unique(rows)
    qr = oracle.quantize("mxfp4", to_f32(W[torch.from_numpy(rows)]))
    wd = oracle.dequant(qr)
    for B in (1, 4, 16):
        x = wl.tensors[f"x{B}"]
        y = torch.empty((B, N), dtype=torch.bfloat16, device=DEV)
        q4.q4_gemv(qg, x.to(DEV), y)
        torch.cuda.synchronize()
        ref = oracle.matmul_f64(to_f32(x), wd)
        e = check_matmul(y.cpu()[:, torch.from_numpy(rows)], ref, to_f32(x), wd, True,
                         f"mxfp4 decode B={B}")
        log("mxfp4 decode gemv B", B, "max normalized error", e)


@pytest.mark.parametrize("fmt", ("int4", "nvfp4", "int4_zp"))
def test_full_decode_gemv_other_formats(fmt):
    """The same 28672 x 8192 decode weight in the other tiled formats the
    benchmark times, B = 1, 4, 16: 256 sampled output columns against the
    oracle (NVFP4 under the oracle's tensor scale of the whole weight)."""
    wl = workloads.mxfp4_gemv()
    W = wl.tensors["W"]
    N, K = W.shape
    log("decode gemv: quantize", fmt)
    qg = q4.quantize(W.to(DEV), fmt, layout="tiled")
    rows = np.sort(np.random.default_rng(29).choice(N, 256, replace=False))
    rows[:3] = [0, N // 2, N - 1]
    rows = np.unique(rows)
    gs = oracle.nv_global_scale(to_f32(W)) if fmt == "nvfp4" else None
    wd = oracle.dequant(oracle.quantize(fmt, to_f32(W[torch.from_numpy(rows)]), gs=gs))
    for B in (1, 4, 16):
        x = wl.tensors[f"x{B}"]
        y = torch.empty((B, N), dtype=torch.bfloat16, device=DEV)
        q4.q4_gemv(qg, x.to(DEV), y)
        torch.cuda.synchronize()
        e = check_matmul(y.cpu()[:, torch.from_numpy(rows)], oracle.matmul_f64(to_f32(x), wd), to_f32(x), wd,
                         EXACT[fmt], f"{fmt} decode B={B}")
        log(fmt, "decode gemv B", B, "max normalized error", e)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("fmt", FMTS)
def test_strided_operands_match_contiguous(fmt, layout):
    """Row strides of x / A and of y / C larger than the rows (column slices
    of wider tensors) give bit for bit the contiguous results: GEMV, W4A16
    GEMM and the grouped GEMM."""
    N, K = 272, 1024
    w = workloads.matrix("tst/w", 4 * N, K, 0.02, seed=61)
    qg, _ = quantized(w, fmt, layout)
    qn, _ = quantized(w[:N], fmt, layout)
    a = workloads.matrix("tst/a", 40, K, 1.0, seed=62).to(DEV)
    wide = torch.full((40, K + 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    wide[:, :K] = a
    a_s = wide[:, :K]
    for B in (1, 16):
        y0 = torch.empty((B, N), dtype=torch.bfloat16, device=DEV)
        y1 = torch.full((B, N + 8), float("nan"), dtype=torch.bfloat16, device=DEV)
        q4.q4_gemv(qn, a[:B].contiguous(), y0)
        q4.q4_gemv(qn, a_s[:B], y1[:, :N])
        torch.cuda.synchronize()
        assert torch.equal(y0, y1[:, :N]) and torch.isnan(y1[:, N:]).all()
    c0 = torch.empty((40, N), dtype=torch.bfloat16, device=DEV)
    c1 = torch.full((40, N + 24), float("nan"), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(a, qn, c0)
    q4.q4_gemm(a_s, qn, c1[:, :N])
    torch.cuda.synchronize()
    assert torch.equal(c0, c1[:, :N]) and torch.isnan(c1[:, N:]).all()
    logits = workloads.normal_f32("tst/l", 40 * 4, seed=63).reshape(40, 4)
    r = workloads.route(logits, 2)
    ga, of = torch.from_numpy(r.gather).to(DEV), torch.from_numpy(r.offsets).to(DEV)
    P = len(r.gather)
    g0 = torch.empty((P, N), dtype=torch.bfloat16, device=DEV)
    g1 = torch.full((P, N + 8), float("nan"), dtype=torch.bfloat16, device=DEV)
    q4.q4_grouped_gemm(a, ga, of, qg, N, g0)
    q4.q4_grouped_gemm(a_s, ga, of, qg, N, g1[:, :N])
    torch.cuda.synchronize()
    assert torch.equal(g0, g1[:, :N]) and torch.isnan(g1[:, N:]).all()
    # odd leading dimensions, and outputs that start at an odd element (2-byte
    # but not 4-byte aligned): the kernels' 4-wide bf16 stores fall back to
    # narrower ones and the results are the same
    for off, extra in ((0, 1), (1, 3)):
        log("strided", fmt, layout, "output offset", off, "ld", N + off + extra)
        c2 = torch.full((40, N + off + extra), float("nan"), dtype=torch.bfloat16, device=DEV)
        q4.q4_gemm(a, qn, c2[:, off:off + N])
        g2 = torch.full((P, N + off + extra), float("nan"), dtype=torch.bfloat16, device=DEV)
        q4.q4_grouped_gemm(a, ga, of, qg, N, g2[:, off:off + N])
        y2 = torch.full((16, N + off + extra), float("nan"), dtype=torch.bfloat16, device=DEV)
        q4.q4_gemv(qn, a[:16].contiguous(), y2[:, off:off + N])
        torch.cuda.synchronize()
        y0 = torch.empty((16, N), dtype=torch.bfloat16, device=DEV)
        q4.q4_gemv(qn, a[:16].contiguous(), y0)
        torch.cuda.synchronize()
        for got, ref in ((c2, c0), (g2, g0), (y2, y0)):
            assert torch.equal(got[:, off:off + N], ref)
            assert torch.isnan(got[:, :off]).all() and torch.isnan(got[:, off + N:]).all()


# --------------------------------------------------------------------------
# W4A16 GEMM
# --------------------------------------------------------------------------
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(200, 300, 512), (64, 256, 128), (1, 1000, 1024), (333, 520, 1152),
                                   (130, 1030, 2048), (256, 512, 4096), (600, 700, 1024)])
def test_gemm_w4a16_small(fmt, M, N, K, layout):
    if layout == "tiled" and not tiled_ok(K):
        pytest.skip("the tiled layout needs K % 512 == 0")
    log("gemm w4a16", fmt, layout, M, N, K)
    w = workloads.matrix(f"tm/w{N}x{K}", N, K, 0.02, seed=31)
    a = workloads.matrix(f"tm/a{M}x{K}", M, K, 1.0, seed=32, channel_frac=0.01, channel_mult=10.0)
    qg, qr = quantized(w, fmt, layout)
    C = torch.full((M, N + 4), float("nan"), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(a.to(DEV), qg, C[:, :N])
    torch.cuda.synchronize()
    Cc = C.cpu()
    assert torch.isnan(Cc[:, N:]).all()
    wd = oracle.dequant(qr)
    check_matmul(Cc[:, :N], oracle.matmul_f64(to_f32(a), wd), to_f32(a), wd, EXACT[fmt],
                 f"w4a16 {fmt}")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_w4a16_tiny_scales(fmt, layout):
    M, N, K = 70, 96, 1024
    w = tiny_rows(N, K, 30)
    a = workloads.matrix("tm/tinya", M, K, 1.0, seed=34)
    qg, qr = quantized(w, fmt, layout)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(a.to(DEV), qg, C)
    torch.cuda.synchronize()
    wd = oracle.dequant(qr)
    check_matmul(C.cpu(), oracle.matmul_f64(to_f32(a), wd), to_f32(a), wd, EXACT[fmt], f"w4a16 tiny {fmt}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_full_nvfp4_prefill_gemm(layout):
    """4096 x 8192 x 8192 with NVFP4 weights: 64 sampled rows of C (all 8192
    columns) against the oracle."""
    wl = workloads.nvfp4_gemm()
    A, W = wl.tensors["A"], wl.tensors["W"]
    M, N = A.shape[0], W.shape[0]
    log("nvfp4 prefill: quantize", layout)
    qg, qr = quantized(W, "nvfp4", layout)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(A.to(DEV), qg, C)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(33).choice(M, 62, replace=False)]))
    wd = oracle.dequant(qr)
    a = to_f32(A[torch.from_numpy(rows)])
    e = check_matmul(C.cpu()[torch.from_numpy(rows)], oracle.matmul_f64(a, wd), a, wd, False,
                     "nvfp4 prefill")
    log("nvfp4 prefill max normalized error", e)


# --------------------------------------------------------------------------
# W4A4 MXFP4 GEMM
# --------------------------------------------------------------------------
@pytest.mark.parametrize("alayout,wlayout", [("rows", "rows"), ("tiled", "tiled"),
                                             ("rows", "tiled"), ("tiled", "rows")])
@pytest.mark.parametrize("M,N,K", [(200, 300, 512), (64, 256, 128), (129, 1000, 1024), (65, 1030, 2048)])
def test_gemm_w4a4_small(M, N, K, alayout, wlayout):
    if "tiled" in (alayout, wlayout) and not tiled_ok(K):
        pytest.skip("the tiled layout needs K % 512 == 0")
    log("gemm w4a4", alayout, wlayout, M, N, K)
    w = workloads.matrix(f"t4/w{N}x{K}", N, K, 0.02, seed=41)
    a = workloads.matrix(f"t4/a{M}x{K}", M, K, 1.0, seed=42)
    qw, qwr = quantized(w, "mxfp4", wlayout)
    qa, qar = quantized(a, "mxfp4", alayout)
    C = torch.full((M, N + 4), float("nan"), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(qa, qw, C[:, :N])
    torch.cuda.synchronize()
    Cc = C.cpu()
    assert torch.isnan(Cc[:, N:]).all()
    ad, wd = oracle.dequant(qar), oracle.dequant(qwr)
    check_matmul(Cc[:, :N], oracle.gemm_w4a4(None, qwr, aq=qar), ad, wd, True, "w4a4")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_w4a4_identity_a_returns_w_transposed(layout):
    K = 512
    w = workloads.matrix("t4/id", 128, K, 0.05, seed=43)
    qw, qwr = quantized(w, "mxfp4", layout)
    qa, _ = quantized(torch.eye(K, dtype=torch.bfloat16), "mxfp4", layout)
    C = torch.empty((K, 128), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(qa, qw, C)
    torch.cuda.synchronize()
    got = C.cpu().float().numpy()
    exp = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(oracle.dequant(qwr).T.copy()))
    assert np.array_equal(got, exp)   # values: -0 and +0 compare equal


def test_full_w4a4_gemm():
    """8192^3 W4A4: A and W quantized on the GPU, 64 sampled rows of C."""
    wl = workloads.w4a4_gemm()
    A, W = wl.tensors["A"], wl.tensors["W"]
    M, N = A.shape[0], W.shape[0]
    log("w4a4: quantize (tiled, the benchmark's layout)")
    qw, qwr = quantized(W, "mxfp4", "tiled")
    qa = q4.quantize(A.to(DEV), "mxfp4", layout="tiled")
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(qa, qw, C)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(44).choice(M, 62, replace=False)]))
    qar = oracle.quantize("mxfp4", to_f32(A[torch.from_numpy(rows)]))
    ad, wd = oracle.dequant(qar), oracle.dequant(qwr)
    e = check_matmul(C.cpu()[torch.from_numpy(rows)], oracle.gemm_w4a4(None, qwr, aq=qar), ad, wd,
                     True, "w4a4 8192")
    log("w4a4 max normalized error", e)


# --------------------------------------------------------------------------
# W4A4 NVFP4 GEMM (both operands NVFP4, each with its own global scale)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("alayout,wlayout", [("rows", "rows"), ("tiled", "tiled"),
                                             ("rows", "tiled"), ("tiled", "rows")])
@pytest.mark.parametrize("M,N,K", [(200, 300, 512), (64, 256, 128), (129, 1000, 1024), (65, 1030, 2048),
                                   (300, 520, 1536)])
def test_gemm_w4a4_nvfp4_small(M, N, K, alayout, wlayout):
    if "tiled" in (alayout, wlayout) and not tiled_ok(K):
        pytest.skip("the tiled layout needs K % 512 == 0")
    log("gemm w4a4 nvfp4", alayout, wlayout, M, N, K)
    w = workloads.matrix(f"t4n/w{N}x{K}", N, K, 0.02, seed=45, outlier_frac=0.001, outlier_mult=20.0)
    a = workloads.matrix(f"t4n/a{M}x{K}", M, K, 1.0, seed=46, channel_frac=0.01, channel_mult=10.0)
    qw, qwr = quantized(w, "nvfp4", wlayout)
    qa, qar = quantized(a, "nvfp4", alayout)
    C = torch.full((M, N + 4), float("nan"), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(qa, qw, C[:, :N])
    torch.cuda.synchronize()
    Cc = C.cpu()
    assert torch.isnan(Cc[:, N:]).all()
    ad, wd = oracle.dequant(qar), oracle.dequant(qwr)
    check_matmul(Cc[:, :N], oracle.gemm_w4a4(None, qwr, aq=qar), ad, wd, True, "w4a4 nvfp4")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_w4a4_nvfp4_identity_a_returns_w_transposed(layout):
    """NVFP4 maps A = I exactly, so C = w'^T within the output rounding."""
    K = 512
    w = tiny_rows(128, K, 47)          # scales spanning six decades, E4M3 subnormals included
    qw, qwr = quantized(w, "nvfp4", layout)
    qa, qar = quantized(torch.eye(K, dtype=torch.bfloat16), "nvfp4", layout)
    assert np.array_equal(oracle.dequant(qar), np.eye(K, dtype=np.float32))
    C = torch.empty((K, 128), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(qa, qw, C)
    torch.cuda.synchronize()
    wd = oracle.dequant(qwr)
    check_matmul(C.cpu(), wd.T.astype(np.float64), np.eye(K, dtype=np.float32), wd, True, "w4a4 nvfp4 I")


def test_w4a4_nvfp4_power_of_two_scaling_of_a():
    """A -> 4A leaves every code and block scale and moves A's global scale
    by 4, so C -> 4C exactly (the global scales enter after the sum)."""
    M, N, K = 128, 256, 1024
    w = workloads.matrix("t4n/pw", N, K, 0.02, seed=48)
    a = workloads.matrix("t4n/pa", M, K, 1.0, seed=49)
    qw, _ = quantized(w, "nvfp4", "tiled")
    out = []
    for f in (1.0, 4.0):
        qa = q4.quantize((a.float() * f).to(torch.bfloat16).to(DEV), "nvfp4", layout="tiled")
        C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        q4.q4_gemm(qa, qw, C)
        out.append(C.float().cpu())
    torch.cuda.synchronize()
    assert torch.equal(out[1], out[0] * 4.0)


def test_full_w4a4_nvfp4_gemm():
    """8192^3 W4A4 with NVFP4 operands (the W4A4 workload's A and W): 64
    sampled rows of C against the oracle (A's global scale from the whole A)."""
    wl = workloads.w4a4_gemm()
    A, W = wl.tensors["A"], wl.tensors["W"]
    M, N = A.shape[0], W.shape[0]
    log("w4a4 nvfp4: quantize (tiled)")
    qw, qwr = quantized(W, "nvfp4", "tiled")
    qa, qar = quantized(A, "nvfp4", "tiled")
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q4.q4_gemm(qa, qw, C)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(50).choice(M, 62, replace=False)]))
    ref = oracle.gemm_w4a4(None, qwr, rows=rows, aq=qar)
    ad = oracle.dequant_rows(qar, rows)
    e = check_matmul(C.cpu()[torch.from_numpy(rows)], ref, ad, oracle.dequant(qwr), True, "w4a4 nvfp4 8192")
    log("w4a4 nvfp4 max normalized error", e)


# --------------------------------------------------------------------------
# grouped MoE GEMM
# --------------------------------------------------------------------------
def _grouped_case(E, N, K, T, topk, seed, fmt="mxfp4"):
    w = workloads.matrix(f"tgr/w{E}x{N}x{K}", E * N, K, 0.02, seed=seed)
    a = workloads.matrix(f"tgr/a{T}x{K}", T, K, 1.0, seed=seed + 1)
    logits = workloads.normal_f32(f"tgr/l{T}x{E}", T * E, seed=seed + 2).reshape(T, E)
    return w, a, workloads.route(logits, topk)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("E,N,K,T,topk", [(8, 200, 512, 50, 2), (16, 128, 256, 300, 4),
                                          (4, 72, 128, 3, 1), (8, 144, 1024, 70, 3),
                                          (4, 272, 512, 300, 2)])   # ~150 rows per expert
def test_grouped_small(fmt, E, N, K, T, topk, layout):
    if layout == "tiled" and not tiled_ok(K, N):
        pytest.skip("the tiled layout needs K % 512 == 0 and N % 16 == 0")
    log("grouped", fmt, layout, E, N, K, T, topk)
    w, a, r = _grouped_case(E, N, K, T, topk, 51)
    qg, qr = quantized(w, fmt, layout)
    P = len(r.gather)
    C = torch.full((P, N + 2), float("nan"), dtype=torch.bfloat16, device=DEV)
    q4.q4_grouped_gemm(a.to(DEV), torch.from_numpy(r.gather).to(DEV),
                       torch.from_numpy(r.offsets).to(DEV), qg, N, C[:, :N])
    torch.cuda.synchronize()
    Cc = C.cpu()
    assert torch.isnan(Cc[:, N:]).all()
    ref = oracle.grouped_gemm(to_f32(a), r.gather, r.offsets, qr, N)
    wd = oracle.dequant(qr)
    af = to_f32(a)
    for e in range(E):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        if hi > lo:
            check_matmul(Cc[lo:hi, :N], ref[lo:hi], af[r.gather[lo:hi]], wd[e * N:(e + 1) * N],
                         EXACT[fmt], f"grouped {fmt} expert {e}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_grouped_empty_experts_and_bad_gather(layout):
    """Experts with no rows are skipped; a gather index outside [0, T)
    produces a zero row; offsets beyond P are clamped."""
    E, N, K, T = 4, 64, 512, 10
    w, a, _ = _grouped_case(E, N, K, T, 1, 61)
    qg, qr = quantized(w, "mxfp4", layout)
    gather = np.array([0, 1, 2, 99, 3, -5, 4], np.int32)     # rows 3 and 5 invalid
    offsets = np.array([0, 3, 3, 7, 7], np.int32)            # experts 1 and 3 empty
    C = torch.full((7, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    q4.q4_grouped_gemm(a.to(DEV), torch.from_numpy(gather).to(DEV),
                       torch.from_numpy(offsets).to(DEV), qg, N, C)
    torch.cuda.synchronize()
    Cc = C.cpu().float().numpy()
    assert np.all(Cc[3] == 0) and np.all(Cc[5] == 0)
    wd = oracle.dequant(qr)
    af = to_f32(a)
    for p, e in [(0, 0), (1, 0), (2, 0), (4, 2), (6, 2)]:
        ref = af[gather[p]].astype(np.float64) @ wd[e * N:(e + 1) * N].astype(np.float64).T
        check_matmul(C.cpu()[p:p + 1], ref[None], af[gather[p]][None], wd[e * N:(e + 1) * N],
                     True, f"row {p}")


def test_full_moe_grouped():
    """64 experts of 2048 x 7168 MXFP4, 256 tokens routed top-8: every routed
    row of eight experts checked against the oracle."""
    wl = workloads.moe_grouped()
    W, A, r = wl.tensors["W"], wl.tensors["A"], wl.meta["routing"]
    N = wl.meta["N"]
    log("moe: quantize (tiled, the benchmark's layout)")
    qg = q4.quantize(W.to(DEV), "mxfp4", layout="tiled")
    P = len(r.gather)
    C = torch.empty((P, N), dtype=torch.bfloat16, device=DEV)
    q4.q4_grouped_gemm(A.to(DEV), torch.from_numpy(r.gather).to(DEV),
                       torch.from_numpy(r.offsets).to(DEV), qg, N, C)
    torch.cuda.synchronize()
    Cc = C.cpu()
    af = to_f32(A)
    worst = 0.0
    for e in (0, 9, 18, 27, 36, 45, 54, 63):
        qr = oracle.quantize("mxfp4", to_f32(W[e * N:(e + 1) * N]))
        wd = oracle.dequant(qr)
        lo, hi = r.offsets[e], r.offsets[e + 1]
        ref = oracle.matmul_f64(af[r.gather[lo:hi]], wd)
        worst = max(worst, check_matmul(Cc[lo:hi], ref, af[r.gather[lo:hi]], wd, True, f"expert {e}"))
    log("moe grouped max normalized error", worst)
