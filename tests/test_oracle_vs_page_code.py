"""The oracle against the pages' own fake-quantization functions.

"Quantization in deployment" (section Fake quantization, the formats.py
listing) defines fp4(), mxfp4() and nvfp4() as torch code that quantizes a
tensor and immediately dequantizes it in fp32; "Low-bit inference for very
large MoE" (section "Why quantization-aware training") defines fake_int4()
the same way.  The page_* functions below compute what those functions
compute, with the same fp32 operations in the same order, written here as
their own torch code; each test asserts that the oracle's quantize followed
by its dequant returns the same fp32 values bit for bit.  This pins the
oracle's fp32 operation order (NVFP4: the block scale E4M3((amax_b / 6) /
gs), the element quotient w / fp32(E4M3 * gs)), not only its formulas.

The oracle departs from those functions only where its readings say so,
and each departure is asserted on its own:
  * exact E2M1 midpoints: fp4() takes an argmin, which returns the smaller
    grid value; the oracle rounds ties to the even code and has a test-only
    switch for the argmin behaviour, on in these comparisons (the E4M3 cast
    and torch.round keep ties to even either way);
  * the INT4 scale is stored in fp16 (g128 with an FP16 scale, "Quantization
    chains", "Bits per weight"), so page_fake_int4 takes fake_int4's scale
    rounded to fp16; a group of zeros, where fake_int4 divides 0 by 0, is 0
    in the oracle;
  * an NVFP4 block whose E4M3 scale rounds to 0: nvfp4() clamps the scale to
    1e-12 before multiplying by gs, so its nonzero values saturate to
    +-6 * fp32(1e-12 * gs); the oracle stores scale 0 and returns 0.

Negative controls show that the inputs can see the slips an oracle could
plausibly make: the NVFP4 block scale as amax_b / (6 gs), the element
quotient as (w / E4M3) / gs, and ties to even in fp4().
"""
import numpy as np
import pytest
import torch

import oracle

F32 = np.float32
GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# what the pages' functions compute, in torch fp32
# --------------------------------------------------------------------------
def page_fp4(x, scale, ties_to_even=False):
    """fp4(): y = clamp(x / scale, -6, 6); the grid value nearest |y| (on an
    exact tie the first, i.e. smaller, one: an argmin over the increasing
    grid); times sign(y), times scale.  ties_to_even is a negative control."""
    y = torch.clamp(x / scale, -6.0, 6.0)
    a = y.abs()
    best = torch.zeros_like(a)
    best_d = (a - GRID[0]).abs()
    for i, v in enumerate(GRID[1:], start=1):
        d = (a - v).abs()
        take = d < best_d
        if ties_to_even:
            take = take | ((d == best_d) & (i % 2 == 0))
        best = torch.where(take, torch.full_like(a, v), best)
        best_d = torch.where(take, d, best_d)
    return best * torch.sign(y) * scale


def page_mxfp4(w, block=32, ties_to_even=False):
    """mxfp4(): blocks of 32 along the last axis; amax clamped at 1e-12;
    scale 2^(floor(log2 amax) - 2); fp4() with that scale."""
    g = w.reshape(w.shape[0], -1, block)
    amax = g.abs().amax(-1, keepdim=True).clamp(min=1e-12)
    scale = torch.exp2(torch.floor(torch.log2(amax)) - 2.0)
    return page_fp4(g, scale, ties_to_even).reshape(w.shape)


def page_nvfp4_global_scale(w):
    """nvfp4()'s tensor scale: max(amax, 1e-12) / (448 * 6), in fp32."""
    return w.abs().max().clamp(min=1e-12) / (E4M3_MAX * 6.0)


def page_nvfp4(w, block=16, gs=None, slip=None):
    """nvfp4(): blocks of 16; block scale = E4M3 cast of (amax_b / 6) / gs;
    fp4() with the scale fp32(max(E4M3, 1e-12) * gs).  `gs` given replaces
    the tensor's own (a caller-supplied tensor scale).  `slip` selects a
    negative control: "scale" computes amax_b / (6 gs), "quotient" divides
    by the E4M3 value first and by gs second."""
    g = w.reshape(w.shape[0], -1, block)
    if gs is None:
        gs = page_nvfp4_global_scale(w)
    gs = torch.as_tensor(gs, dtype=torch.float32)
    amax_b = g.abs().amax(-1, keepdim=True)
    if slip == "scale":
        t = amax_b / (6.0 * gs)
    else:
        t = amax_b / 6.0 / gs
    bs = t.to(torch.float8_e4m3fn).float()
    if slip == "quotient":
        v = page_fp4(g / bs.clamp(min=1e-12), gs)
        return v.reshape(w.shape)
    return page_fp4(g, bs.clamp(min=1e-12) * gs).reshape(w.shape)


def page_fake_int4(w, group=128):
    """fake_int4(): symmetric INT4 per group of input channels; scale amax / 7
    (here rounded to fp16, the stored scale); round half to even, clamp to
    [-8, 7], times the scale."""
    g = w.reshape(w.shape[0], -1, group)
    s = (g.abs().amax(-1, keepdim=True) / 7.0).half().float()
    q = torch.round(g / s).clamp(-8, 7) * s
    return q.reshape(w.shape)


# --------------------------------------------------------------------------
# inputs
# --------------------------------------------------------------------------
def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=F32)).bfloat16().float().numpy()


def _weights(rows, cols, seed, std, outlier_frac, outlier_mult):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((rows, cols)) * std).astype(F32)
    n = int(round(outlier_frac * w.size))
    w.ravel()[rng.choice(w.size, n, replace=False)] *= F32(outlier_mult)
    return _bf16(w)


def _random_cases():
    """bf16 weights like the workloads' (normal, a fraction of outliers),
    at several non-power-of-two magnitudes so that gs takes many values."""
    out = []
    for i, (std, frac, mult) in enumerate([(0.02, 0.001, 20.0), (0.015, 0.0005, 30.0),
                                           (1.0, 0.0, 1.0), (0.37, 0.01, 10.0),
                                           (3.1e-3, 0.002, 7.0), (45.0, 0.001, 3.3)]):
        out.append(_weights(32, 2048, 100 + i, std, frac, mult))
    return out


def _near(x, ulps):
    """x moved by `ulps` fp32 ulps (x > 0)."""
    b = np.asarray(x, dtype=F32).view(np.uint32).astype(np.int64) + ulps
    return b.astype(np.uint32).view(F32)


def _boundary_rows_mx(rng, rows):
    """fp32 blocks of 32 whose quotients w / 2^e sit exactly on, and a few
    ulps either side of, every E2M1 midpoint and the saturation at 6.  Each
    block's largest value is a bf16 number whose exponent fixes e, so no
    block maximum lies an ulp below a power of two (where an fp32 log2
    rounds up to the integer: for bf16 inputs that cannot happen)."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    w = np.zeros((rows, 32 * 8), dtype=F32)
    for r in range(rows):
        for b in range(8):
            e = int(rng.integers(-20, 10))
            blk = []
            for m in mids:
                for u in (-2, -1, 0, 1, 2):
                    v = _near(F32(m) * F32(2.0 ** e), u) if u else F32(m * 2.0 ** e)
                    blk.append(v)
            blk = np.array(blk[:31], dtype=F32)
            blk *= np.where(rng.random(31) < 0.5, F32(-1), F32(1))
            # block max: 6.5 * 2^e, a bf16 value in [4, 8) * 2^e -> scale 2^e
            w[r, 32 * b:32 * b + 32] = np.concatenate([blk, [F32(6.5 * 2.0 ** e)]])
    return w


def _e4m3_value(code):
    return float(torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).float())


def _boundary_rows_nv(rng, rows, gs):
    """fp32 blocks of 16 for a fixed tensor scale gs: each block's largest
    value puts (amax_b / 6) / gs on, or a few ulps off, an E4M3 midpoint, and
    the other values put w / fp32(E4M3 * gs) on, or a few ulps off, an E2M1
    midpoint of the E4M3 value the block's scale rounds to."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    w = np.zeros((rows, 16 * 16), dtype=F32)
    gs = F32(gs)
    for r in range(rows):
        for b in range(16):
            code = int(rng.integers(0x09, 0x7E))           # E4M3 value and its neighbour up
            lo, hi = _e4m3_value(code), _e4m3_value(code + 1)
            mid = F32((lo + hi) / 2)                        # exact in fp32
            amax = F32(F32(mid * gs) * F32(6.0))
            amax = _near(amax, int(rng.integers(-2, 3)))
            t = F32(F32(amax / F32(6.0)) / gs)
            s = torch.tensor([float(t)]).to(torch.float8_e4m3fn).float().item()
            eff = F32(F32(s) * gs)
            vals = []
            for k in range(15):
                m = F32(mids[k % len(mids)])
                v = _near(F32(m * eff), int(rng.integers(-3, 4)))
                vals.append(min(v, amax))
            vals = np.array(vals, dtype=F32) * np.where(rng.random(15) < 0.5, F32(-1), F32(1))
            w[r, 16 * b:16 * b + 16] = np.concatenate([vals, [amax]])
    return w


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------
@pytest.fixture
def argmin_ties():
    oracle.set_ties_toward_zero(True)
    try:
        yield
    finally:
        oracle.set_ties_toward_zero(False)


def _oracle_fake(fmt, w, gs=None):
    return oracle.dequant(oracle.quantize(fmt, w, gs=gs))


def _page(fn, w, **kw):
    return fn(torch.from_numpy(np.ascontiguousarray(w, dtype=F32)), **kw).numpy()


def _same_bits(a, b):
    """Equal fp32 values, compared as bits; zeros of either sign compare
    equal (fp4() multiplies by sign(y), which is +0 for y = -0)."""
    a = np.asarray(a, dtype=F32)
    b = np.asarray(b, dtype=F32)
    same = a.view(np.uint32) == b.view(np.uint32)
    return same | ((a == 0) & (b == 0))


# --------------------------------------------------------------------------
# MXFP4
# --------------------------------------------------------------------------
def test_mxfp4_matches_page_code_random(argmin_ties):
    for w in _random_cases():
        got = _oracle_fake("mxfp4", w)
        ref = _page(page_mxfp4, w)
        assert np.all(_same_bits(got, ref))


def test_mxfp4_matches_page_code_at_boundaries(argmin_ties):
    w = _boundary_rows_mx(np.random.default_rng(7), 16)
    assert np.all(_same_bits(_oracle_fake("mxfp4", w), _page(page_mxfp4, w)))


def test_mxfp4_control_ties_to_even_is_seen():
    """Without the switch (the oracle's reading, ties to even) the oracle and
    fp4()'s argmin part on exact midpoints, which bf16 weights hit often
    under a power-of-two scale: the inputs above contain them."""
    w = _random_cases()[0]
    got = _oracle_fake("mxfp4", w)
    ref = _page(page_mxfp4, w)
    diff = ~_same_bits(got, ref)
    assert diff.sum() > 0
    # ... and exactly those elements agree with the ties-to-even variant
    ref_even = _page(page_mxfp4, w, ties_to_even=True)
    assert np.all(_same_bits(got, ref_even))


# --------------------------------------------------------------------------
# NVFP4
# --------------------------------------------------------------------------
def test_nvfp4_matches_page_code_random(argmin_ties):
    for w in _random_cases():
        got = _oracle_fake("nvfp4", w)
        ref = _page(page_nvfp4, w)
        q = oracle.quantize("nvfp4", w)
        assert F32(q.gs) == _page(page_nvfp4_global_scale, w)
        under = np.repeat(q.scales == 0, 16, axis=1)
        assert np.all(_same_bits(got, ref)[~under])


@pytest.mark.parametrize("gs", [1.0, 3.7e-4, 0.0123, 2.9e-6, 171.3])
def test_nvfp4_matches_page_code_at_boundaries(argmin_ties, gs):
    """Block scales on and a few ulps off E4M3 midpoints, element quotients
    on and off E2M1 midpoints, under a caller-supplied tensor scale (the
    page's function with its gs replaced by the given one)."""
    w = _boundary_rows_nv(np.random.default_rng(int(gs * 1e6) % 1000 + 11), 8, gs)
    got = _oracle_fake("nvfp4", w, gs=gs)
    ref = _page(page_nvfp4, w, gs=F32(gs))
    assert np.all(_same_bits(got, ref))


@pytest.mark.parametrize("gs", [3.7e-4, 2.9e-6, 171.3])
def test_nvfp4_controls_swapped_operation_order_are_seen(gs):
    """An oracle that computed amax_b / (6 gs), or (w / E4M3) / gs, would
    fail the comparison above: the page's function with that slip differs
    from the oracle on these inputs."""
    oracle.set_ties_toward_zero(True)
    try:
        w = _boundary_rows_nv(np.random.default_rng(int(gs * 1e6) % 1000 + 11), 8, gs)
        got = _oracle_fake("nvfp4", w, gs=gs)
        for slip in ("scale", "quotient"):
            ref = _page(page_nvfp4, w, gs=F32(gs), slip=slip)
            assert (~_same_bits(got, ref)).sum() > 0, slip
    finally:
        oracle.set_ties_toward_zero(False)


# Two blocks where the order of the NVFP4 block-scale divisions decides the
# E4M3 code, with a tensor scale that is not a power of two.  Worked in fp32:
#   gs = 0x3c1b82c8 (0.00949163), amax_b = 0x3cf7d870 (0.030254573):
#     fp32(amax_b / 6) / gs = 0.53125 exactly, the midpoint of E4M3 0.5 (0x30)
#     and 0.5625 (0x31): ties to even give 0x30;
#     amax_b / fp32(6 gs) = 0.53125006, above the midpoint: 0x31.
#   gs = 0x3b860c46 (0.0040908186), amax_b = 0x3bd5a390 (0.0065197423):
#     the page's order gives 0.26562503, above the midpoint of 0.25 (0x28) and
#     0.28125 (0x29): 0x29; the swapped order gives 0.265625, a tie: 0x28.
ORDER_CASES = [(0x3c1b82c8, 0x3cf7d870, 0x30, 0x31), (0x3b860c46, 0x3bd5a390, 0x29, 0x28)]


def _f32_from_bits(b):
    return np.array([b], dtype=np.uint32).view(F32)[0]


@pytest.mark.parametrize("gs_bits,amax_bits,code,swapped_code", ORDER_CASES)
def test_nvfp4_block_scale_operation_order_worked_cases(gs_bits, amax_bits, code, swapped_code):
    gs, amax = _f32_from_bits(gs_bits), _f32_from_bits(amax_bits)
    assert oracle.nv_block_scale_code(float(amax), float(gs)) == code
    t = torch.tensor([float(amax)]) / 6.0 / torch.tensor([float(gs)])
    assert int(t.to(torch.float8_e4m3fn).view(torch.uint8)) == code
    t_swapped = torch.tensor([float(amax)]) / (6.0 * torch.tensor([float(gs)]))
    assert int(t_swapped.to(torch.float8_e4m3fn).view(torch.uint8)) == swapped_code
    # the whole block through quantize: the stored code and the page function
    W = np.zeros((1, 16), dtype=F32)
    W[0, 0] = amax
    W[0, 1] = -F32(0.5) * amax
    q = oracle.quantize("nvfp4", W, gs=float(gs))
    assert int(q.scales[0, 0]) == code
    oracle.set_ties_toward_zero(True)
    try:
        assert np.all(_same_bits(oracle.dequant(q), _page(page_nvfp4, W, gs=gs)))
    finally:
        oracle.set_ties_toward_zero(False)


def test_nvfp4_underflowing_block_scale_reading():
    """Blocks whose (amax_b / 6) / gs is below half the smallest E4M3
    subnormal (2^-10): the oracle stores scale 0 and returns 0 for every
    value; nvfp4() clamps the scale at 1e-12, so its nonzero values become
    +-6 * fp32(1e-12 * gs) and its zeros stay 0.  Both dequantize the block
    to within 6e-12 gs of 0."""
    rng = np.random.default_rng(3)
    w = _bf16(rng.standard_normal((4, 64)).astype(F32))
    w[:, :16] *= F32(1e-5)           # tiny blocks next to a large tensor amax
    w[0, 16] = F32(300.0)
    q = oracle.quantize("nvfp4", w)
    gs = F32(q.gs)
    assert np.all(q.scales[:, 0] == 0)
    got = oracle.dequant(q)
    ref = _page(page_nvfp4, w)
    assert np.all(got[:, :16] == 0)
    floor = F32(F32(1e-12) * gs)
    expect = np.where(w[:, :16] == 0, F32(0), np.sign(w[:, :16]) * F32(6.0) * floor)
    assert np.array_equal(ref[:, :16], expect.astype(F32))
    oracle.set_ties_toward_zero(True)
    try:
        got = oracle.dequant(oracle.quantize("nvfp4", w))
    finally:
        oracle.set_ties_toward_zero(False)
    assert np.all(_same_bits(got, ref)[:, 16:])


# --------------------------------------------------------------------------
# INT4 (fake_int4 with its scale stored in fp16)
# --------------------------------------------------------------------------
def test_int4_matches_page_code_random():
    for w in _random_cases():
        got = _oracle_fake("int4", w)
        ref = _page(page_fake_int4, w)
        assert np.all(_same_bits(got, ref))


def test_int4_matches_page_code_at_ties():
    """Quotients exactly on half-integers (torch.round sends them to the even
    integer, as the oracle does) and a few ulps either side of them."""
    rng = np.random.default_rng(9)
    rows = []
    for _ in range(8):
        s = F32(rng.uniform(1e-3, 1.0))
        s = F32(torch.tensor([float(s)]).half().float().item())
        amax = F32(7.0) * s                       # fp16(amax / 7) = s again
        vals = []
        for k in range(127):
            h = F32((k % 15) - 7 + 0.5)
            v = F32(h * s)
            vals.append(_near(abs(v), int(rng.integers(-2, 3))) * np.sign(v) if v != 0 else v)
        row = np.concatenate([np.array(vals, dtype=F32), [amax]])
        rows.append(np.clip(row, -amax, amax))
    w = np.stack(rows).astype(F32)
    got = _oracle_fake("int4", w)
    ref = _page(page_fake_int4, w)
    assert np.all(_same_bits(got, ref))


def test_int4_zero_group_reading():
    """A group of zeros: fake_int4 computes 0 / 0 (NaN); the oracle stores
    scale 0 and returns 0.  The other groups of the row still match."""
    w = _weights(2, 512, 5, 0.02, 0.0, 1.0)
    w[:, 128:256] = 0.0
    got = _oracle_fake("int4", w)
    ref = _page(page_fake_int4, w)
    assert np.all(np.isnan(ref[:, 128:256]))
    assert np.all(got[:, 128:256] == 0)
    keep = np.ones(512, dtype=bool)
    keep[128:256] = False
    assert np.all(_same_bits(got[:, keep], ref[:, keep]))
