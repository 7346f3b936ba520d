"""GPU parity of q4_quantize / q4_dequant against the oracle: packed codes,
scales and the NVFP4 global scale bit for bit; dequantized values bit for
bit (fp32 and bf16)."""
import numpy as np
import pytest
import torch

import oracle
import w4_gemm_amd as q4
from w4_gemm_amd import workloads
from q4_helpers import assert_quant_equal, log, to_f32

pytestmark = pytest.mark.gpu
FMTS = ("int4", "mxfp4", "nvfp4", "int4_zp")
DEV = "cuda:0"


def quant_both(w_bf16: torch.Tensor, fmt: str, gs=None, layout="rows"):
    wd = w_bf16.to(DEV)
    gs_t = None if gs is None else torch.tensor([gs], dtype=torch.float32, device=DEV)
    qg = q4.quantize(wd, fmt, nv_global_in=gs_t, layout=layout)
    torch.cuda.synchronize()
    qr = oracle.quantize(fmt, to_f32(w_bf16), gs=gs)
    return qg, qr


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(1, 128), (3, 256), (37, 640), (130, 1024), (257, 384)])
def test_quantize_small_random(fmt, shape):
    log("quantize", fmt, shape)
    rows, cols = shape
    w = workloads.matrix(f"tq/{rows}x{cols}", rows, cols, 0.02, seed=11,
                         outlier_frac=0.002, outlier_mult=25.0)
    qg, qr = quant_both(w, fmt)
    assert_quant_equal(qg, qr, fmt)


@pytest.mark.parametrize("fmt,shape", [("mxfp4", (5, 96)), ("mxfp4", (33, 224)), ("nvfp4", (3, 48)),
                                       ("nvfp4", (40, 208))])
def test_quantize_row_major_short_rows(fmt, shape):
    """Row lengths that are not a multiple of 128 (MXFP4 % 32, NVFP4 % 16):
    the lane-per-8-values quantizer."""
    log("quantize short rows", fmt, shape)
    rows, cols = shape
    w = workloads.matrix(f"tq/{rows}x{cols}", rows, cols, 0.02, seed=12,
                         outlier_frac=0.01, outlier_mult=25.0)
    qg, qr = quant_both(w, fmt)
    assert_quant_equal(qg, qr, fmt)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(1, 512), (16, 512), (37, 1024), (130, 1536), (257, 512)])
def test_quantize_small_random_tiled(fmt, shape):
    log("quantize tiled", fmt, shape)
    rows, cols = shape
    w = workloads.matrix(f"tq/t{rows}x{cols}", rows, cols, 0.02, seed=17,
                         outlier_frac=0.002, outlier_mult=25.0)
    qg, qr = quant_both(w, fmt, layout="tiled")
    assert_quant_equal(qg, qr, fmt)
    # the padding rows of the last tile hold the quantization of zeros
    pad = (-rows) % 16
    if pad:
        zq = oracle.quantize(fmt, np.zeros((16, cols), np.float32))
        from q4_helpers import scales_np, untile
        c, sc = untile(qg.codes.cpu().numpy(), scales_np(qg, fmt), fmt, rows + pad, cols)
        assert np.array_equal(c[rows:], zq.codes[:pad]) and np.array_equal(sc[rows:], zq.scales[:pad])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("layout", ("rows", "tiled"))
def test_quantize_all_bf16_values(fmt, layout):
    """Every finite bf16 bit pattern, grouped into blocks in three different
    orders so each value meets many block scales."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = v[np.isfinite(v)]
    if fmt in ("int4", "int4_zp"):
        v = v[np.abs(v) < 4e5]  # fp16 scale range (|w| < 7*65504; (hi - lo)/15 < 65504)
    rng = np.random.default_rng(12)
    for order in ("sorted", "shuffled", "mixed"):
        x = v.copy()
        if order == "shuffled":
            rng.shuffle(x)
        elif order == "mixed":  # small values next to a large one in each block
            x = np.sort(np.abs(x))[::-1].copy() * np.where(rng.random(x.size) < 0.5, -1, 1)
            x = x[: (x.size // 16) * 16].reshape(-1, 16)[:, ::-1].reshape(-1).copy()
        n = (x.size // 1024) * 1024
        w = torch.from_numpy(x[:n].reshape(-1, 1024)).to(torch.bfloat16)
        log("all bf16", fmt, layout, order, tuple(w.shape))
        qg, qr = quant_both(w, fmt, layout=layout)
        assert_quant_equal(qg, qr, fmt)


@pytest.mark.parametrize("fmt", ("mxfp4", "nvfp4"))
def test_quantize_exact_ties(fmt):
    """Values that land exactly on E2M1 midpoints (0.25, 0.75, ... 5) after
    the division: ties go to the even code on both sides."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    rows = []
    for e in range(-6, 6):
        blk = np.zeros(32, np.float32)
        blk[0] = 6.0 * 2.0 ** e           # absmax -> scale 2^(e)  (floor(log2 6) - 2 = 0)
        blk[1:8] = mids * 2.0 ** e
        blk[8:15] = -mids * 2.0 ** e
        rows.append(blk)
    w = torch.from_numpy(np.stack(rows)).to(torch.bfloat16)
    if fmt == "nvfp4":
        qg, qr = quant_both(w, fmt, gs=1.0)
    else:
        qg, qr = quant_both(w, fmt)
    assert_quant_equal(qg, qr, fmt)


@pytest.mark.parametrize("fmt", ("int4", "int4_zp"))
@pytest.mark.parametrize("layout", ("rows", "tiled"))
def test_int4_exact_ties(fmt, layout):
    """Half-integer quotients as exact ties: -6.5 .. 6.5 (INT4), -7.5 .. 6.5
    and, with a zero point of -4, -3.5 .. 10.5 (INT4 with zero point).  Each
    group's scale is a power of two (INT4: absmax 7 2^e; zero point: range
    [lo, hi] with (hi - lo) / 15 = 2^e), and the values are (k + 1/2) 2^e."""
    rows = []
    for e in range(-10, 10):
        for lo_k, hi_k in ((-8, 7), (-4, 11)):
            if fmt == "int4" and lo_k != -8:
                continue
            ks = np.arange(-7 if fmt == "int4" else lo_k, 7 if fmt == "int4" else hi_k, dtype=np.float32)
            ties = (ks + 0.5) * np.float32(2.0 ** e)
            g = np.resize(np.concatenate([ties, -ties if fmt == "int4" else ties]), 128).astype(np.float32)
            if fmt == "int4":
                g[0] = 7.0 * 2.0 ** e      # absmax -> s = fp16(7 2^e / 7) = 2^e
            else:
                g[0], g[1] = lo_k * 2.0 ** e, hi_k * 2.0 ** e
            rows.append(np.concatenate([g, g[::-1], g[::-1], g]))  # 512: a tiled row
    x = np.stack(rows)
    w = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(to_f32(w), x)
    log("int4 ties", fmt, layout, tuple(w.shape))
    qg, qr = quant_both(w, fmt, layout=layout)
    assert_quant_equal(qg, qr, fmt)


@pytest.mark.parametrize("cols", (128, 48))
def test_nvfp4_quotients_next_to_rounding_boundaries(cols):
    """NVFP4 quotients a few ulp either side of every E2M1 rounding boundary.
    With the caller's tensor scale gs = 1 + k 2^-23 and a block whose absmax
    is 6v (v an E4M3 value), the block scale is v and w = b v divides to
    b / gs: within |k| ulp of the boundary b.  The code is the rounding of
    the fp32 quotient, so this is where a shortcut around the division would
    have to be exact.  cols 128 takes the block-mapped kernel, 48 the
    per-chunk one."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    vs = np.array([m / 8.0 * 2.0 ** e for e in range(-6, 8) for m in range(8, 16)], np.float32)
    blocks = np.zeros((vs.size, 16), np.float32)
    blocks[:, 0] = 6.0 * vs
    blocks[:, 1:8] = mids[None, :] * vs[:, None]
    blocks[:, 8:15] = -mids[None, :] * vs[:, None]
    per_row = cols // 16
    n = (blocks.shape[0] // per_row) * per_row
    w = torch.from_numpy(blocks[:n].reshape(-1, cols)).to(torch.bfloat16)
    assert np.array_equal(to_f32(w).reshape(-1, 16), blocks[:n])  # every value exact in bf16
    for k in (-40, -12, -6, -3, -2, -1, 0, 1, 2, 3, 6, 12, 40):
        gs = float(np.float32(1.0 + k * 2.0 ** -23))
        log("nvfp4 near boundaries", cols, k)
        qg, qr = quant_both(w, "nvfp4", gs=gs)
        assert_quant_equal(qg, qr, "nvfp4")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("layout", ("rows", "tiled"))
def test_quantize_edge_blocks(fmt, layout):
    w = np.zeros((8, 512), np.float32)
    w[1] = -0.0
    w[2, :] = 1e-30                      # below the 1e-12 clamp
    w[3, ::2] = 3.0e38                   # near the top of fp32 (MX, NV only)
    w[4, :] = np.float32(2.0 ** -130)    # bf16 subnormal
    w[5, 7] = 1.0                        # one nonzero per block
    w[6, :] = np.linspace(-1, 1, 512)
    w[7, :] = 448.0 * 6 * np.sign(np.linspace(-1, 1, 512))
    if fmt in ("int4", "int4_zp"):
        w[3] = 0.0
        w[7] = np.sign(w[7]) * 1000.0
    wt = torch.from_numpy(w).to(torch.bfloat16)
    qg, qr = quant_both(wt, fmt, layout=layout)
    assert_quant_equal(qg, qr, fmt)


def test_nvfp4_caller_global_scale_and_underflow():
    w = workloads.matrix("tq/nv", 64, 512, 0.02, seed=13)
    for gs in (1.0, 0.001, 1e-6, 3.0):
        qg, qr = quant_both(w, "nvfp4", gs=gs)
        assert_quant_equal(qg, qr, "nvfp4")
    # a tiny block next to a large tensor max: its E4M3 scale underflows to 0
    x = np.zeros((2, 32), np.float32)
    x[0, 0] = 100.0
    x[1, :16] = 1e-6
    x[1, 16:] = -1e-6
    qg, qr = quant_both(torch.from_numpy(x).to(torch.bfloat16), "nvfp4")
    assert_quant_equal(qg, qr, "nvfp4")
    assert np.all(qr.scales[1] == 0)


def test_quantize_strided_source_and_empty():
    base = workloads.matrix("tq/strided", 40, 1024, 0.05, seed=14)
    view = base[:, :512]                          # ld = 1024 > cols
    for fmt in FMTS:
        qg = q4.quantize(base.to(DEV)[:, :512], fmt)
        torch.cuda.synchronize()
        qr = oracle.quantize(fmt, to_f32(view))
        assert_quant_equal(qg, qr, fmt)
    e = q4.empty_q4("nvfp4", 0, 128, device=DEV)
    q4.q4_quantize(torch.empty((0, 128), dtype=torch.bfloat16, device=DEV), e)
    torch.cuda.synchronize()
    assert e.global_scale.item() == np.float32(1e-12) / np.float32(2688.0)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("layout,rows,cols", [("rows", 96, 768), ("rows", 97, 896), ("tiled", 90, 1024)])
def test_dequant_bit_exact(fmt, layout, rows, cols):
    w = workloads.matrix(f"tq/dq{cols}", rows, cols, 0.03, seed=15, outlier_frac=0.01,
                         outlier_mult=30.0)
    qg, qr = quant_both(w, fmt, layout=layout)
    ref = oracle.dequant(qr)
    out32 = torch.full((rows, cols + 8), float("nan"), device=DEV)
    q4.q4_dequant(qg, out32[:, :cols])
    out16 = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    q4.q4_dequant(qg, out16)
    torch.cuda.synchronize()
    o32 = out32.cpu().numpy()
    assert np.array_equal(o32[:, :cols].view(np.uint32), ref.view(np.uint32))
    assert np.all(np.isnan(o32[:, cols:]))        # nothing written past cols
    o16 = out16.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o16, oracle.f32_to_bf16_bits(ref))


def test_quantize_deterministic():
    w = workloads.matrix("tq/det", 512, 2048, 0.02, seed=16).to(DEV)
    for fmt in FMTS:
        a, b = q4.quantize(w, fmt), q4.quantize(w, fmt)
        torch.cuda.synchronize()
        assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)


# --------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark uses
# --------------------------------------------------------------------------
def check_dequant_sampled(qg, qr, nrows=64, seed=5):
    """The GPU dequantization of the whole tensor (bf16 and fp32) against the
    oracle's on sampled rows (the first, the last and random ones), bit for
    bit."""
    rows, cols = qr.rows, qr.cols
    rng = np.random.default_rng(seed)
    pick = np.unique(np.concatenate([[0, rows - 1], rng.integers(0, rows, nrows - 2)]))
    ref = oracle.dequant_rows(qr, pick)
    d16 = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    q4.q4_dequant(qg, d16)
    got16 = d16[torch.from_numpy(pick).to(DEV)].cpu().float().numpy()
    del d16
    exp16 = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(ref))
    assert np.array_equal(got16.view(np.uint32), exp16.view(np.uint32))
    d32 = torch.empty((rows, cols), dtype=torch.float32, device=DEV)
    q4.q4_dequant(qg, d32)
    got32 = d32[torch.from_numpy(pick).to(DEV)].cpu().numpy()
    del d32
    assert np.array_equal(got32.view(np.uint32), ref.view(np.uint32))


def test_full_int4_gemv_weight():
    wl = workloads.int4_gemv()
    qg, qr = quant_both(wl.tensors["W"], "int4")
    assert_quant_equal(qg, qr, "int4")
    check_dequant_sampled(qg, qr)


@pytest.mark.parametrize("layout", ("rows", "tiled"))
def test_full_mxfp4_decode_weight(layout):
    wl = workloads.mxfp4_gemv(batches=(1,))
    log("quantize 28672x8192 MXFP4", layout)
    qg, qr = quant_both(wl.tensors["W"], "mxfp4", layout=layout)
    assert_quant_equal(qg, qr, "mxfp4")
    log("dequantize 28672x8192 MXFP4 (sampled rows)", layout)
    check_dequant_sampled(qg, qr)


@pytest.mark.parametrize("layout", ("rows", "tiled"))
def test_full_nvfp4_prefill_weight(layout):
    wl = workloads.nvfp4_gemm()
    log("quantize 8192x8192 NVFP4", layout)
    qg, qr = quant_both(wl.tensors["W"], "nvfp4", layout=layout)
    assert_quant_equal(qg, qr, "nvfp4")
    log("dequantize 8192x8192 NVFP4 (sampled rows)", layout)
    check_dequant_sampled(qg, qr)


def test_full_w4a4_operands():
    wl = workloads.w4a4_gemm()
    for name in ("A", "W"):
        log("quantize 8192x8192 MXFP4 tiled", name)
        qg, qr = quant_both(wl.tensors[name], "mxfp4", layout="tiled")
        assert_quant_equal(qg, qr, "mxfp4")


def test_full_moe_experts_weight():
    """All 64 experts quantized in one call on the GPU; the oracle checks
    four of them completely."""
    wl = workloads.moe_grouped()
    W = wl.tensors["W"]
    N = wl.meta["N"]
    log("quantize 64x2048x7168 MXFP4 tiled")
    qg = q4.quantize(W.to(DEV), "mxfp4", layout="tiled")
    torch.cuda.synchronize()
    for e in (0, 21, 42, 63):
        rows = np.arange(e * N, (e + 1) * N)
        qr = oracle.quantize("mxfp4", to_f32(W[e * N:(e + 1) * N]))
        assert_quant_equal(qg, qr, "mxfp4", rows=rows)


@pytest.mark.parametrize("fmt", ("int4", "nvfp4", "int4_zp"))
def test_full_decode_weight_other_formats(fmt):
    """The other formats the benchmark quantizes at 28672 x 8192 (tiled): the
    codes and scales of 256 sampled rows, read back row-major through the
    layout conversion, bit for bit against the oracle (NVFP4: also the
    tensor scale, from the oracle over the whole weight)."""
    wl = workloads.mxfp4_gemv(batches=(1,))
    W = wl.tensors["W"]
    N = W.shape[0]
    log("quantize 28672x8192 tiled", fmt)
    qg = q4.quantize(W.to(DEV), fmt, layout="tiled")
    qrow = q4.relayout(qg, "rows")
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(31).choice(N, 254, replace=False)]))
    gs = oracle.nv_global_scale(to_f32(W)) if fmt == "nvfp4" else None
    qr = oracle.quantize(fmt, to_f32(W[torch.from_numpy(rows)]), gs=gs)
    sel = torch.from_numpy(rows).to(DEV)
    codes = qrow.codes[sel].cpu().numpy()
    scales = qrow.scales[sel].cpu().contiguous().view(torch.uint8).numpy()
    assert np.array_equal(codes, qr.codes)
    assert np.array_equal(scales, np.ascontiguousarray(qr.scales).view(np.uint8).reshape(scales.shape))
    if fmt == "nvfp4":
        assert np.float32(qg.global_scale.item()).view(np.uint32) == np.float32(gs).view(np.uint32)
