"""Pins of the oracle's matmul references (fp64 on dequantized weights).

Brute force on tiny inputs (explicit Python loops), special cases with a
closed form, and the grouped GEMM against a per-expert dense product.
"""
import numpy as np

import oracle
from w4_gemm_amd import workloads


def _w(rows, cols, seed, std=0.02):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, cols)) * std).astype(np.float32)


def test_gemv_matches_explicit_loops():
    w = _w(5, 128, 1)
    x = np.random.default_rng(2).standard_normal((3, 128)).astype(np.float32)
    for fmt in ("int4", "mxfp4", "nvfp4"):
        q = oracle.quantize(fmt, w)
        d = oracle.dequant(q)
        ref = oracle.gemv(q, x)
        for b in range(3):
            for n in range(5):
                s = 0.0
                for k in range(128):
                    s += float(x[b, k]) * float(d[n, k])
                assert abs(ref[b, n] - s) <= 1e-12 * max(1.0, abs(s))


def test_one_hot_x_selects_a_dequantized_column():
    w = _w(7, 256, 3)
    for fmt in ("int4", "mxfp4", "nvfp4"):
        q = oracle.quantize(fmt, w)
        d = oracle.dequant(q)
        for k in (0, 17, 255):
            x = np.zeros((1, 256), np.float32)
            x[0, k] = 1.0
            assert np.array_equal(oracle.gemv(q, x)[0], d[:, k].astype(np.float64))


def test_all_ones_accumulates_exactly():
    """All-ones MXFP4 weights times an all-ones x over K = 1024 give exactly
    1024 (a bf16 running sum would stop at 256)."""
    w = np.ones((4, 1024), np.float32)
    q = oracle.quantize("mxfp4", w)
    assert np.all(oracle.dequant(q) == 1.0)
    assert np.all(oracle.gemv(q, np.ones((1, 1024), np.float32)) == 1024.0)


def test_w4a4_identity_a_gives_w_transposed():
    """A = I is exactly representable in MXFP4 (1.0 and zero blocks), so
    C = I . w'^T = w'^T."""
    k = 128
    w = _w(64, k, 4)
    q = oracle.quantize("mxfp4", w)
    a = np.eye(k, dtype=np.float32)
    c = oracle.gemm_w4a4(a, q)
    assert np.array_equal(c, oracle.dequant(q).T.astype(np.float64))


def test_w4a4_quantizes_a_like_the_weights():
    a = _w(16, 256, 5, std=1.0)
    w = _w(32, 256, 6)
    qa, qw = oracle.quantize("mxfp4", a), oracle.quantize("mxfp4", w)
    ref = oracle.dequant(qa).astype(np.float64) @ oracle.dequant(qw).astype(np.float64).T
    assert np.array_equal(oracle.gemm_w4a4(a, qw), ref)
    assert np.array_equal(oracle.gemm_w4a4(a, qw, rows=[3, 9]), ref[[3, 9]])


def _e2m1_from_bits(nib):
    """E2M1 nibble -> value from its bit fields (sign bit 3, exponent bits
    2:1, mantissa bit 0; exponent 0 is the subnormal 0 / 0.5)."""
    e, m = (nib >> 1) & 3, nib & 1
    mag = 0.5 * m if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)
    return -mag if nib & 8 else mag


def _e4m3_from_bits(b):
    e, m = (b >> 3) & 0xF, b & 7
    return m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)


def _nvfp4_decode(q):
    """Dequantize an NVFP4 QTensor from the bit fields: fp32(code * fp32(E4M3 * gs))."""
    out = np.zeros((q.rows, q.cols), np.float32)
    for r in range(q.rows):
        for k in range(q.cols):
            byte = int(q.codes[r, k // 2])
            nib = byte & 0xF if k % 2 == 0 else byte >> 4
            eff = np.float32(np.float32(_e4m3_from_bits(int(q.scales[r, k // 16]))) * np.float32(q.gs))
            out[r, k] = np.float32(np.float32(_e2m1_from_bits(nib)) * eff)
    return out


def test_w4a4_nvfp4_matches_explicit_loops():
    """W4A4 NVFP4: both operands NVFP4 (E4M3 per 16, each its own tensor
    scale); the reference against a decode written from the bit fields and
    explicit loops."""
    a = _w(3, 64, 11, std=1.0)
    a[1, 5] = 30.0                                   # an outlier sets A's global scale
    w = _w(4, 64, 12)
    qa, qw = oracle.quantize("nvfp4", a), oracle.quantize("nvfp4", w)
    da, dw = _nvfp4_decode(qa), _nvfp4_decode(qw)
    ref = oracle.gemm_w4a4(a, qw)
    for m in range(3):
        for n in range(4):
            s = 0.0
            for k in range(64):
                s += float(da[m, k]) * float(dw[n, k])
            assert abs(ref[m, n] - s) <= 1e-12 * max(1.0, abs(s))


def test_w4a4_nvfp4_identity_a_gives_w_transposed():
    """NVFP4 maps I exactly (a lone 1.0 gets E4M3 448 and code 6, and
    fp32(6 * fp32(448 * gs)) = 1 for gs = 1/2688; zero blocks are zero), so
    C = w'^T."""
    k = 128
    q = oracle.quantize("nvfp4", _w(64, k, 13))
    a = np.eye(k, dtype=np.float32)
    assert np.array_equal(oracle.dequant(oracle.quantize("nvfp4", a)), a)
    assert np.array_equal(oracle.gemm_w4a4(a, q), oracle.dequant(q).T.astype(np.float64))


def test_w4a4_nvfp4_power_of_two_scaling_of_a():
    """A -> 2^j A moves A's global scale by 2^j and leaves every code and
    E4M3 block scale unchanged, so C -> 2^j C exactly."""
    a = _w(8, 256, 14, std=1.0)
    qw = oracle.quantize("nvfp4", _w(16, 256, 15))
    c = oracle.gemm_w4a4(a, qw)
    for j in (-3, 5):
        qa2 = oracle.quantize("nvfp4", a * np.float32(2.0 ** j))
        qa = oracle.quantize("nvfp4", a)
        assert np.array_equal(qa2.codes, qa.codes) and np.array_equal(qa2.scales, qa.scales)
        assert np.array_equal(oracle.gemm_w4a4(a * np.float32(2.0 ** j), qw), c * 2.0 ** j)


def test_w4a4_nvfp4_rows_use_the_whole_a_global_scale():
    a = _w(16, 256, 16, std=1.0)
    a[12, 7] = 50.0                                  # outside the selected rows
    qw = oracle.quantize("nvfp4", _w(32, 256, 17))
    full = oracle.gemm_w4a4(a, qw)
    assert np.array_equal(oracle.gemm_w4a4(a, qw, rows=[3, 9]), full[[3, 9]])
    qa = oracle.quantize("nvfp4", a)
    assert np.array_equal(oracle.gemm_w4a4(None, qw, rows=[3, 9], aq=qa), full[[3, 9]])


def test_grouped_matches_per_expert_dense():
    E, N, K, T, topk = 6, 24, 256, 20, 2
    w = _w(E * N, K, 7)
    a = np.random.default_rng(8).standard_normal((T, K)).astype(np.float32)
    logits = np.random.default_rng(9).standard_normal((T, E)).astype(np.float32)
    r = workloads.route(logits, topk)
    q = oracle.quantize("mxfp4", w)
    out = oracle.grouped_gemm(a, r.gather, r.offsets, q, N)
    d = oracle.dequant(q).astype(np.float64)
    for t in range(T):
        for e in r.topk_ids[t]:
            # the routed row of (t, e)
            lo, hi = r.offsets[e], r.offsets[e + 1]
            p = lo + list(r.gather[lo:hi]).index(t)
            assert np.array_equal(out[p], a[t].astype(np.float64) @ d[e * N:(e + 1) * N].T)
