"""Pins of the oracle's MoE layer pieces (routing, SwiGLU, combine, the
whole layer) against library routines, closed forms, brute force and
invariants -- none of them re-uses the oracle's own code path."""
import numpy as np
import scipy.special

import oracle


def test_routing_matches_stable_argsort_and_softmax():
    rng = np.random.default_rng(1)
    T, E, k = 37, 16, 4
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[3, :] = 0.5                      # all tied: the lowest ids win
    lg[5, [2, 9]] = lg[5].max() + 1.0   # a tie for first place
    r = oracle.moe_route(lg, k)
    ids = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    assert np.array_equal(r.ids, ids)
    assert list(r.ids[3]) == [0, 1, 2, 3] and list(r.ids[5][:2]) == [2, 9]
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(r.weights, np.take_along_axis(p, ids, axis=1), rtol=1e-12, atol=0)
    assert np.allclose(r.weights[3], 1.0 / E)


def test_routing_dispatch_is_expert_major_token_ascending():
    rng = np.random.default_rng(2)
    T, E, k = 50, 8, 3
    lg = rng.standard_normal((T, E)).astype(np.float32)
    r = oracle.moe_route(lg, k)
    counts = np.array([(r.ids == e).sum() for e in range(E)])
    assert list(r.offsets) == [0] + list(np.cumsum(counts))
    for e in range(E):
        toks = sorted(t for t in range(T) if e in r.ids[t])
        assert list(r.gather[r.offsets[e]:r.offsets[e + 1]]) == toks
    for t in range(T):
        for j in range(k):
            p = r.inv[t, j]
            e = r.ids[t, j]
            assert r.gather[p] == t and r.offsets[e] <= p < r.offsets[e + 1]
    assert sorted(r.inv.ravel()) == list(range(T * k))


def test_silu_and_swiglu():
    z = np.linspace(-30, 30, 2001)
    assert np.allclose(oracle.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    assert np.allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=0, atol=1e-12)
    assert oracle.silu(0.0) == 0.0
    gu = np.array([[1.0, -2.0, 3.0, 0.5]])
    h = oracle.swiglu(gu, 2)
    assert np.allclose(h, [[3.0 / (1 + np.exp(-1.0)), 0.5 * -2.0 / (1 + np.exp(2.0))]], rtol=1e-15)


def test_combine_brute_force():
    rng = np.random.default_rng(3)
    T, k, N = 6, 3, 5
    y = rng.standard_normal((T * k, N))
    inv = rng.permutation(T * k).reshape(T, k)
    w = rng.random((T, k))
    out = oracle.moe_combine(y, inv, w)
    for t in range(T):
        for n in range(N):
            assert abs(out[t, n] - sum(w[t, j] * y[inv[t, j], n] for j in range(k))) < 1e-13


def _ffn(x, wg, wu, wd):
    g = wg @ x
    u = wu @ x
    return wd @ (g * scipy.special.expit(g) * u)


def test_moe_layer_one_expert_is_the_dense_ffn():
    rng = np.random.default_rng(4)
    K, I, T = 512, 128, 3
    wgu = (rng.standard_normal((2 * I, K)) * 0.05).astype(np.float32)
    wd = (rng.standard_normal((K, I)) * 0.05).astype(np.float32)
    qgu, qd = oracle.quantize("mxfp4", wgu), oracle.quantize("mxfp4", wd)
    x = rng.standard_normal((T, K)).astype(np.float32)
    out, r = oracle.moe_layer(x, np.zeros((T, 1), dtype=np.float32), 1, qgu, qd, I)
    assert np.all(r.weights == 1.0)
    g_u = oracle.dequant(qgu).astype(np.float64)
    d = oracle.dequant(qd).astype(np.float64)
    for t in range(T):
        ref = _ffn(x[t].astype(np.float64), g_u[:I], g_u[I:], d)
        assert np.allclose(out[t], ref, rtol=1e-12, atol=1e-12)


def test_moe_layer_identical_experts_sum_to_one_ffn():
    """With every expert holding the same weights and k = E, the gates are
    the full softmax, which sums to 1: the layer equals one dense FFN."""
    rng = np.random.default_rng(5)
    E, K, I, T = 4, 512, 64, 5
    wgu = (rng.standard_normal((2 * I, K)) * 0.05).astype(np.float32)
    wd = (rng.standard_normal((K, I)) * 0.05).astype(np.float32)
    qgu = oracle.quantize("mxfp4", np.tile(wgu, (E, 1)))
    qd = oracle.quantize("mxfp4", np.tile(wd, (E, 1)))
    x = rng.standard_normal((T, K)).astype(np.float32)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    out, r = oracle.moe_layer(x, lg, E, qgu, qd, I)
    assert np.allclose(r.weights.sum(axis=1), 1.0, rtol=1e-14)
    g_u = oracle.dequant(oracle.quantize("mxfp4", wgu)).astype(np.float64)
    d = oracle.dequant(oracle.quantize("mxfp4", wd)).astype(np.float64)
    for t in range(T):
        assert np.allclose(out[t], _ffn(x[t].astype(np.float64), g_u[:I], g_u[I:], d), rtol=1e-10, atol=1e-12)
