"""Pins of the oracle's INT4 with a zero point (one fp16 scale and one zero
point per 128 values; "Quantization in deployment", format cheat sheet, row
W4A16 INT4 GPTQ/AWQ): a group built so that every step is exact, the
one-signed and all-zero special cases, exactness of 0, the half-step error
bound, and a brute-force nearest-grid check of every code."""
import numpy as np

import oracle


def _word(scale_bits, z):
    return scale_bits | ((z & 0xFF) << 16)


def test_exact_arithmetic_group():
    c = 2.0 ** -4                                   # fp16 0x2C00
    k = np.arange(128) % 16
    w = ((k - 5) * c).astype(np.float32)            # lo = -5c, hi = 10c: range 15c, scale c
    word, q = oracle.int4zp_group(w)
    assert word == _word(0x2C00, -3)                # z = -8 - rne(-5) = -3
    assert np.array_equal(q, k - 8)
    d = oracle.dequant(oracle.quantize("int4_zp", w.reshape(1, -1)))
    assert np.array_equal(d[0], w)                  # every value on the grid


def test_one_signed_and_zero_groups():
    rng = np.random.default_rng(1)
    pos = np.abs(rng.standard_normal(128)).astype(np.float32)
    word, q = oracle.int4zp_group(pos)
    assert (word >> 16) & 0xFF == 0xF8              # z = -8: code -8 is 0
    assert q.min() >= -8 and q.max() == 7
    neg = -pos
    word, q = oracle.int4zp_group(neg)
    assert (word >> 16) & 0xFF == 7                 # z = 7: code 7 is 0
    assert q.max() <= 7 and q.min() == -8
    word, q = oracle.int4zp_group(np.zeros(128, dtype=np.float32))
    assert word == 0 and not q.any()


def _groups(seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((64, 128)).astype(np.float32) * 0.02 + rng.standard_normal((64, 1)).astype(np.float32) * 0.05
    w[::7, 3] = 0.0                                  # zeros inside groups
    w[5, 10] *= 40.0                                 # an outlier
    return w


def test_zero_is_exact_and_half_step_bound():
    w = _groups(2)
    q = oracle.quantize("int4_zp", w.reshape(8, -1))
    d = oracle.dequant(q).reshape(64, 128)
    s = np.array([oracle.fp16_value(int(x) & 0xFFFF) for x in q.scales.ravel()], dtype=np.float64).reshape(64, 1)
    assert np.all(d[w == 0.0] == 0.0)
    assert np.all(np.abs(d.astype(np.float64) - w) <= s / 2 * (1 + 1e-6))


def test_codes_are_the_nearest_grid_points():
    w = _groups(3)
    for row in w:
        word, q = oracle.int4zp_group(row)
        s = oracle.fp16_value(word & 0xFFFF)
        zb = (word >> 16) & 0xFF
        z = zb - 256 if zb >= 128 else zb
        grid = (np.arange(-8, 8) - z) * np.float64(s)           # value of codes -8..7
        for x, code in zip(row.astype(np.float64), q):
            dist = np.abs(grid - np.float64(np.float32(x) / np.float32(s)) * s)
            best = np.flatnonzero(dist == dist.min())
            # nearest code; on an exact tie the even (x / s rounded half-to-even) one
            assert code + 8 in best, (x, code, best - 8)
