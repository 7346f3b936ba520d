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
