"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties one part of the oracle to something other than itself:
values printed on the pages (tests/golden/*.json, each with its source),
library routines that implement a piece exactly (torch's float8_e4m3fn cast,
fp16 cast, half-to-even round), brute force on small inputs, and invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def nib(codes_row, k):
    b = int(codes_row[k // 2])
    return b & 0xF if k % 2 == 0 else b >> 4


# --------------------------------------------------------------------------
# the worked example of eight weights
# --------------------------------------------------------------------------
def test_worked_example_int4_scale_and_codes():
    g = golden("worked_example_8_weights.json")
    w = np.array(g["printed"]["weights"], dtype=np.float32)
    code, q = oracle.absmax_int_group(w, 7)
    s = oracle.fp16_value(code)
    assert abs(s - g["printed"]["scale_int4"]) < 5e-5          # 0.88/7 = 0.1257
    assert code == g["derived_by_hand"]["int4_fp16_scale_bits"]
    assert list(q) == g["derived_by_hand"]["int4_codes"]
    i = g["printed"]["weights"].index(g["printed"]["int4_zero_weight"])
    assert q[i] == 0                                            # 0.03 rounds to zero
    # the packed tensor carries the same codes (two's complement nibbles)
    W = np.zeros((1, 128), dtype=np.float32)
    W[0, :8] = w
    qt = oracle.quantize("int4", W)
    assert qt.scales[0, 0] == code
    got = [(n - 16 if n >= 8 else n) for n in (nib(qt.codes[0], k) for k in range(8))]
    assert got == list(q)


def test_worked_example_int8_same_absmax_rule():
    g = golden("worked_example_8_weights.json")["printed"]
    w = np.array(g["weights"], dtype=np.float32)
    code, q = oracle.absmax_int_group(w, 127)
    s = oracle.fp16_value(code)
    assert abs(s - g["scale_int8"]) < 5e-6                       # 0.88/127 = 0.00693
    assert np.all(np.abs(w - q * s) < g["int8_max_abs_error"])  # every weight within 0.003


def test_worked_example_nvfp4_effective_scale_and_051():
    g = golden("worked_example_8_weights.json")
    p, d = g["printed"], g["derived_by_hand"]
    W = np.zeros((1, 16), dtype=np.float32)
    W[0, :8] = p["weights"]
    qt = oracle.quantize("nvfp4", W)
    assert qt.gs == np.float32(np.float32(0.88) / np.float32(2688.0))
    assert qt.scales[0, 0] == d["nvfp4_block_scale_code"]       # E4M3 448
    eff = np.float32(oracle.e4m3_value(int(qt.scales[0, 0]))) * np.float32(qt.gs)
    assert abs(eff - p["scale_fp4"]) < 5e-5                      # 0.88/6 = 0.1467
    mags = [nib(qt.codes[0], k) & 7 for k in range(8)]
    assert mags == d["nvfp4_magnitude_codes"]
    deq = oracle.dequant(qt)[0, :8]
    i = p["weights"].index(p["fp4_weight"])
    lo, hi = p["fp4_neighbours"]
    assert abs(deq[i] - lo) < 5e-3                               # 0.51 -> 0.44
    assert abs(4 * eff - hi) < 5e-3                              # next value up 0.59
    assert abs((p["fp4_weight"] - deq[i]) - p["fp4_loss"]) < 5e-3  # loses 0.07
    # signs follow the weights
    for k, wv in enumerate(p["weights"]):
        assert (nib(qt.codes[0], k) >> 3) == (1 if wv < 0 else 0)


def test_worked_example_mxfp4():
    g = golden("worked_example_8_weights.json")["derived_by_hand"]
    w = golden("worked_example_8_weights.json")["printed"]["weights"]
    W = np.zeros((1, 32), dtype=np.float32)
    W[0, :8] = w
    qt = oracle.quantize("mxfp4", W)
    assert qt.scales[0, 0] == g["mxfp4_e8m0"]
    assert [nib(qt.codes[0], k) & 7 for k in range(8)] == g["mxfp4_magnitude_codes"]
    assert list(oracle.dequant(qt)[0, :8]) == g["mxfp4_dequant"]


def test_outlier_sets_int4_scale():
    g = golden("outlier_sets_int4_scale.json")["printed"]
    w = np.full(128, g["others_magnitude"], dtype=np.float32)
    w[1::2] *= -1
    w[5] = g["outlier"]
    w[10] = 0.1139   # just below half the scale: rounds to zero
    w[11] = 0.1149   # just above: rounds to one step
    code, q = oracle.absmax_int_group(w, 7)
    s = oracle.fp16_value(code)
    assert abs(s - g["int4_scale"]) < 5e-4                      # 1.6/7 = 0.229
    assert abs(s / 2 - g["zero_threshold"]) < 5e-4              # 0.114
    assert q[10] == 0 and q[11] == 1
    small = np.abs(w) < s / 2
    assert np.all(q[small] == 0)                                 # the +-0.1 weights vanish


# --------------------------------------------------------------------------
# E4M3 (NVFP4 block scale)
# --------------------------------------------------------------------------
def test_e4m3_limits():
    g = golden("e4m3_chains.json")["printed"]
    values = [oracle.e4m3_value(c) for c in range(127)]
    assert max(values) == g["e4m3_max"] == oracle.e4m3_value(0x7E)
    positive = [v for v in values if v > 0]
    assert min(positive) == 2.0 ** g["e4m3_min_subnormal_log2"]
    assert oracle.e4m3_value(0x08) == 2.0 ** g["e4m3_min_normal_log2"]
    # three mantissa bits: the step after 1.0 is 2^-3, unit roundoff 2^-4
    one = oracle.e4m3_code(1.0)
    assert oracle.e4m3_value(one + 1) - 1.0 == 2.0 * 2.0 ** g["e4m3_unit_roundoff_log2"]
    assert all(values[i] < values[i + 1] for i in range(126))


def test_e4m3_one_outlier_sets_the_scale():
    g = golden("e4m3_chains.json")["printed"]
    scale = np.float32(g["tensor_absmax"]) / np.float32(g["e4m3_max"])
    assert abs(scale - g["tensor_scale"]) < 5e-4
    v1 = oracle.e4m3_value(oracle.e4m3_code(np.float32(g["small_value"]) / scale)) * scale
    assert v1 == g["small_value_stored"]                          # 0.0002 -> 0
    v2 = oracle.e4m3_value(oracle.e4m3_code(np.float32(g["second_value"]) / scale)) * scale
    assert abs(v2 - g["second_value_stored"]) < 5e-7              # 0.0004 -> 0.000436
    assert round(abs(v2 - g["second_value"]) / g["second_value"] * 100) == g["second_value_error_pct"]
    bscale = np.float32(g["block_absmax"]) / np.float32(g["e4m3_max"])
    for x in (g["small_value"], g["second_value"]):
        v = oracle.e4m3_value(oracle.e4m3_code(np.float32(x) / bscale)) * bscale
        assert round(abs(v - x) / x * 100, 1) == g["block_error_pct"]   # 4.1 %


def _bf16_values(lo, hi):
    bits = np.arange(0, 0x7F80, dtype=np.uint32)  # all finite non-negative bf16
    v = (bits << 16).view(np.float32)
    return v[(v >= lo) & (v <= hi)]


def test_e4m3_encoder_matches_torch_float8_e4m3fn():
    vals = _bf16_values(0.0, 448.0)
    rng = np.random.default_rng(1)
    rnd = (rng.random(200_000) * 448).astype(np.float32)
    tiny = (rng.random(50_000) * 0.02).astype(np.float32)
    # exact midpoints between neighbouring E4M3 values (ties to even)
    ev = np.array([oracle.e4m3_value(c) for c in range(127)], dtype=np.float64)
    mids = ((ev[:-1] + ev[1:]) / 2).astype(np.float32)
    allv = np.concatenate([vals, rnd, tiny, mids])
    ref = torch.from_numpy(allv).to(torch.float8_e4m3fn).float().numpy()
    L = oracle.lib()
    got = np.array([L.oracle_e4m3_value(L.oracle_e4m3_code(float(v))) for v in allv],
                   dtype=np.float32)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# FP16 (INT4 scale) and half-to-even integer rounding
# --------------------------------------------------------------------------
def test_fp16_encoder_matches_torch_half():
    vals = _bf16_values(0.0, 65504.0)
    rng = np.random.default_rng(2)
    rnd = np.concatenate([(rng.random(100_000) * 2.0 ** rng.integers(-30, 16, 100_000))]).astype(np.float32)
    allv = np.concatenate([vals, rnd[rnd <= 65504]])
    ref = torch.from_numpy(allv).half().float().numpy()
    L = oracle.lib()
    got = np.array([L.oracle_fp16_value(L.oracle_fp16_code(float(v))) for v in allv],
                   dtype=np.float32)
    assert np.array_equal(got, ref)
    assert oracle.fp16_code(65520.0) == 0x7C00 and oracle.fp16_code(65519.0) == 0x7BFF


def test_int4_codes_match_half_even_round_and_clamp():
    rng = np.random.default_rng(3)
    for trial in range(200):
        w = (rng.standard_normal(128) * rng.choice([0.02, 1.0, 30.0])).astype(np.float32)
        if trial % 4 == 0:  # force exact .5 ties: w = (j + 0.5) * s for a representable s
            s0 = np.float32(oracle.fp16_value(oracle.fp16_code(np.abs(w).max() / np.float32(7))))
            j = rng.integers(-7, 7, 16)
            w[:16] = ((j + 0.5) * np.float64(s0)).astype(np.float32)
        code, q = oracle.absmax_int_group(w, 7)
        s = torch.tensor(np.abs(w).max() / np.float32(7)).half().float()
        assert oracle.fp16_value(code) == s.item()
        ref = torch.round(torch.from_numpy(w) / s).clamp(-8, 7).int().numpy()
        assert np.array_equal(q, ref)


# --------------------------------------------------------------------------
# E2M1 rounding: brute force
# --------------------------------------------------------------------------
def test_e2m1_nearest_even_brute_force():
    # every finite bf16 value in [0, 8] (clamped to 6 first, as the method does)
    vals = _bf16_values(0.0, 8.0)
    for v in vals:
        a = min(float(v), 6.0)
        c = oracle.e2m1_code(a)
        d = abs(a - E2M1[c])
        dists = [abs(a - g) for g in E2M1]
        assert d == min(dists)
        ties = [i for i, x in enumerate(dists) if x == d]
        if len(ties) > 1:
            assert c % 2 == 0 and c in ties


def test_e2m1_ties_switch_reproduces_first_index_argmin():
    """With the test-only switch, exact midpoints go to the lower neighbour,
    which is what an argmin over the increasing grid returns."""
    mids = [(E2M1[i] + E2M1[i + 1]) / 2 for i in range(7)]
    try:
        oracle.set_ties_toward_zero(True)
        assert [oracle.e2m1_code(m) for m in mids] == list(range(7))
    finally:
        oracle.set_ties_toward_zero(False)
    assert [oracle.e2m1_code(m) for m in mids] == [0, 2, 2, 4, 4, 6, 6]


# --------------------------------------------------------------------------
# MXFP4 / NVFP4 on a block whose largest value is 5.0
# --------------------------------------------------------------------------
def test_block_max_5_mxfp4_vs_nvfp4():
    g = golden("mxfp4_vs_nvfp4_block_max_5.json")["printed"]
    W = np.zeros((1, 32), dtype=np.float32)
    W[0, 0] = g["block_max"]
    W[0, 1] = 1.0
    mx = oracle.quantize("mxfp4", W)
    assert 2.0 ** (int(mx.scales[0, 0]) - 127) == g["mxfp4_scale"]
    v = oracle.dequant(mx)[0, 0]
    assert v == g["mxfp4_stored"]
    assert round(abs(v - 5.0) / 5.0 * 100) == g["mxfp4_error_pct"]
    # NVFP4 with the tensor scale fixed to 1: the block scale is E4M3(5/6)
    nv = oracle.quantize("nvfp4", W[:, :16], gs=1.0)
    assert oracle.e4m3_value(int(nv.scales[0, 0])) == g["nvfp4_scale"]
    assert round(5.0 / g["nvfp4_scale"], 2) == g["nvfp4_quotient"]
    assert E2M1[nib(nv.codes[0], 0) & 7] == g["nvfp4_code_value"]
    v = oracle.dequant(nv)[0, 0]
    assert v == g["nvfp4_stored"]
    assert round(abs(v - 5.0) / 5.0 * 100, 1) == g["nvfp4_error_pct"]


def test_mx_power_of_two_scale_leaves_max_in_4_to_8():
    """MXFP4's scale 2^(floor(log2 amax) - 2) divides a block's maximum down
    to some value in [4, 8), never more than a factor two from the top of
    the E2M1 range ("Quantization chains", "MXFP4 against NVFP4 scales")."""
    rng = np.random.default_rng(4)
    amax = (rng.random(20000) * 2.0 ** rng.integers(-20, 20, 20000)).astype(np.float32) + 1e-9
    for a in amax[:5000]:
        e = oracle.mx_scale_exponent(float(a))
        r = float(a) / 2.0 ** e
        assert 4.0 <= r < 8.0


# --------------------------------------------------------------------------
# sizes: bits per weight
# --------------------------------------------------------------------------
def test_bits_per_weight():
    g = golden("bits_per_weight.json")["printed"]
    rows, cols = 4, 1024
    W = np.zeros((rows, cols), dtype=np.float32)
    for fmt in ("int4", "mxfp4", "nvfp4"):
        q = oracle.quantize(fmt, W)
        bits = 8 * (q.codes.nbytes + q.scales.nbytes) / (rows * cols)
        assert bits == g["bits_per_weight"][fmt]
    assert 0.5 + 1 / 32 == g["bytes_per_param"]["mxfp4"]
    assert 0.5 + 1 / 16 == g["bytes_per_param"]["nvfp4"]


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def _rand(rows, cols, seed, std=0.02):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((rows, cols)) * std).astype(np.float32)
    w.ravel()[rng.choice(w.size, w.size // 500, replace=False)] *= 25
    return w


def test_mx_power_of_two_scale_invariance():
    w = _rand(16, 256, 5)
    q0 = oracle.quantize("mxfp4", w)
    for j in (-5, -1, 1, 7):
        qj = oracle.quantize("mxfp4", w * np.float32(2.0 ** j))
        assert np.array_equal(qj.codes, q0.codes)
        assert np.array_equal(qj.scales.astype(int), q0.scales.astype(int) + j)


def test_sign_symmetry():
    w = _rand(8, 512, 6)
    for fmt in ("int4", "mxfp4", "nvfp4"):
        a, b = oracle.quantize(fmt, w), oracle.quantize(fmt, -w)
        assert np.array_equal(a.scales, b.scales)
        assert np.array_equal(oracle.dequant(a), -oracle.dequant(b))
        if fmt != "int4":
            assert np.array_equal(a.codes ^ 0x88, b.codes)   # E2M1: only the sign bits flip


def test_idempotence_int4_mx():
    w = _rand(8, 512, 7)
    for fmt in ("int4", "mxfp4"):
        q1 = oracle.quantize(fmt, w)
        q2 = oracle.quantize(fmt, oracle.dequant(q1))
        assert np.array_equal(q1.codes, q2.codes) and np.array_equal(q1.scales, q2.scales)


def test_error_bounds():
    """|w - w'| is at most half a grid step times the scale (no clipping by
    construction of absmax scales), except the saturating MXFP4 top range."""
    w = _rand(8, 1024, 8)
    q = oracle.quantize("int4", w)
    d = oracle.dequant(q)
    s = np.repeat(np.array([[oracle.fp16_value(int(c)) for c in row] for row in q.scales]), 128, 1)
    assert np.all(np.abs(w - d) <= s / 2 * (1 + 2.0 ** -10))
    q = oracle.quantize("mxfp4", w)
    d = oracle.dequant(q)
    s = np.repeat(2.0 ** (q.scales.astype(np.float64) - 127), 32, 1)
    y = np.abs(w) / s
    gap = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    ok = np.abs(np.abs(w) - np.abs(d)) / s <= gap / 2
    sat = y > 6
    assert np.all(ok | sat)
    assert np.all(np.abs(d[sat]) == 6 * s[sat])


def test_zero_blocks_and_negative_zero():
    w = np.zeros((2, 128), dtype=np.float32)
    w[1, :] = -0.0
    for fmt in ("int4", "mxfp4", "nvfp4"):
        q = oracle.quantize(fmt, w)
        assert np.all(oracle.dequant(q) == 0)
        if fmt == "int4":
            assert np.all(q.codes == 0) and np.all(q.scales == 0)
        else:
            assert np.all(q.codes[0] == 0) and np.all(q.codes[1] == 0x88)
    assert np.all(oracle.quantize("mxfp4", w).scales == 85)   # 2^-42: amax clamped at 1e-12


def test_nvfp4_block_scale_underflow_gives_zero_codes():
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0] = 1.0
    w[0, 16:] = 1e-9        # (1e-9/6)/(1/2688) < 2^-10: E4M3 scale 0
    w[0, 17] = -1e-9
    q = oracle.quantize("nvfp4", w)
    assert q.scales[0, 1] == 0
    assert nib(q.codes[0], 16) == 0 and nib(q.codes[0], 17) == 8
    assert np.all(oracle.dequant(q)[0, 16:] == 0)


def test_global_scale_definition():
    w = _rand(4, 64, 9)
    gs = oracle.nv_global_scale(w)
    assert gs == np.float32(np.abs(w).max()) / np.float32(2688.0)
    assert oracle.nv_global_scale(np.zeros((2, 16), np.float32)) == np.float32(1e-12) / np.float32(2688)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(10)
    x = (rng.standard_normal(200_000) * 2.0 ** rng.integers(-40, 40, 200_000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits(x), ref)
