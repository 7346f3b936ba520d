"""GPU parity of the MoE layer steps around the grouped GEMM (q4_moe_route,
q4_swiglu, q4_moe_combine) and of the whole layer chained through the C ABI
(route -> gate/up grouped GEMM -> SwiGLU -> down grouped GEMM -> combine),
against the oracle's plain definitions.

Tolerances: routing is exact (ids, offsets, gather, inv) and the gates agree
with the fp64 softmax to 2e-6 relative (fp32 exp and sum).  SwiGLU and the
combine round to bf16 once: |got - ref| <= 2^-8 |ref| + 2^-16 * scale.  The
layer rounds three intermediate products to bf16 (gate/up, h, expert
output) before the fp32 combine: per token, ||out - ref||_2 <= 1e-2 ||ref||_2
and every element within 3e-2 max|ref| (measured errors are reported)."""
import numpy as np
import pytest
import torch

import oracle
import w4_gemm_amd as q4
from w4_gemm_amd import workloads
from q4_helpers import log, to_f32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _logits(T, E, seed):
    lg = workloads.normal_f32(f"tmoe/l{T}x{E}", T * E, seed=seed).reshape(T, E).copy()
    if T > 3:
        lg[1, :] = 0.25                         # all experts tied
        lg[3, : min(E, 4)] = lg[3].max() + 1.0  # a tie for first place
    return lg


@pytest.mark.parametrize("T,E,k", [(256, 64, 8), (37, 16, 4), (1, 8, 8), (0, 8, 2), (1000, 128, 6),
                                   (5, 1024, 32), (300, 70, 3)])
def test_route_exact(T, E, k):
    log("route", T, E, k)
    lg = _logits(T, E, seed=81) if T else np.zeros((0, E), dtype=np.float32)
    r = q4.q4_moe_route(torch.from_numpy(lg).to(DEV), k)
    torch.cuda.synchronize()
    assert list(r.offsets.cpu().numpy()) == ([0] * (E + 1) if T == 0 else list(oracle.moe_route(lg, k).offsets))
    if T == 0:
        return
    ref = oracle.moe_route(lg, k)
    assert np.array_equal(r.ids.cpu().numpy(), ref.ids)
    assert np.array_equal(r.gather.cpu().numpy(), ref.gather)
    assert np.array_equal(r.inv.cpu().numpy(), ref.inv)
    w = r.weights.cpu().numpy().astype(np.float64)
    assert np.allclose(w, ref.weights, rtol=2e-6, atol=1e-30)


def test_route_strided_logits():
    T, E, k = 50, 32, 4
    lg = _logits(T, E + 8, seed=82)
    r = q4.q4_moe_route(torch.from_numpy(lg).to(DEV)[:, :E], k)
    torch.cuda.synchronize()
    ref = oracle.moe_route(np.ascontiguousarray(lg[:, :E]), k)
    assert np.array_equal(r.ids.cpu().numpy(), ref.ids) and np.array_equal(r.inv.cpu().numpy(), ref.inv)


@pytest.mark.parametrize("P,I", [(100, 256), (1, 8), (2048, 2048), (7, 520)])
def test_swiglu(P, I):
    log("swiglu", P, I)
    gu = workloads.matrix(f"tmoe/gu{P}x{I}", P, 2 * I + 8, 2.0, seed=83)
    gu[0, :8] = torch.tensor([0.0, -0.0, 40.0, -40.0, 1e-30, -1e-30, 3.0, -3.0]).bfloat16()
    h = q4.q4_swiglu(gu.to(DEV), I)
    torch.cuda.synchronize()
    ref = oracle.swiglu(to_f32(gu)[:, :2 * I], I)
    got = to_f32(h).astype(np.float64)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-38
    bad = np.argwhere(np.abs(got - ref) > bound)
    assert bad.size == 0, bad[:5].tolist()


@pytest.mark.parametrize("T,E,k,N", [(256, 64, 8, 7168), (37, 16, 4, 512), (3, 8, 1, 64)])
def test_combine(T, E, k, N):
    log("combine", T, E, k, N)
    lg = _logits(T, E, seed=84)
    r = q4.q4_moe_route(torch.from_numpy(lg).to(DEV), k)
    y = workloads.matrix(f"tmoe/y{T}x{k}x{N}", T * k, N, 1.0, seed=85)
    out = q4.q4_moe_combine(y.to(DEV), r)
    torch.cuda.synchronize()
    ref_r = oracle.moe_route(lg, k)
    ref = oracle.moe_combine(to_f32(y), ref_r.inv, ref_r.weights)
    scale = np.einsum("tj,tjn->tn", ref_r.weights, np.abs(to_f32(y).astype(np.float64))[ref_r.inv])
    got = to_f32(out).astype(np.float64)
    bad = np.argwhere(np.abs(got - ref) > 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * scale + 1e-30)
    assert bad.size == 0, bad[:5].tolist()


def _check_layer(out, ref, what):
    got = to_f32(out).astype(np.float64)
    assert np.all(np.isfinite(got))
    for t in range(ref.shape[0]):
        nrm = np.linalg.norm(ref[t])
        e2 = np.linalg.norm(got[t] - ref[t])
        assert e2 <= 1e-2 * nrm, (what, t, e2 / nrm)
        assert np.abs(got[t] - ref[t]).max() <= 3e-2 * np.abs(ref[t]).max(), (what, t)
    rel = max(np.linalg.norm(got[t] - ref[t]) / np.linalg.norm(ref[t]) for t in range(ref.shape[0]))
    log(what, "max relative error per token", rel)


@pytest.mark.parametrize("layout", ("rows", "tiled"))
@pytest.mark.parametrize("fmt", ("mxfp4", "int4", "nvfp4", "int4_zp"))
def test_moe_layer_small(fmt, layout):
    E, I, K, T, k = 8, 512, 1024, 37, 2
    log("moe layer", fmt, layout, E, I, K, T, k)
    wgu = workloads.matrix("tmoe/wgu", E * 2 * I, K, 0.03, seed=86)
    wd = workloads.matrix("tmoe/wd", E * K, I, 0.03, seed=87)
    x = workloads.matrix("tmoe/x", T, K, 1.0, seed=88)
    lg = _logits(T, E, seed=89)
    qgu = q4.quantize(wgu.to(DEV), fmt, layout=layout)
    qd = q4.quantize(wd.to(DEV), fmt, layout=layout)
    out, r = q4.moe_layer(x.to(DEV), torch.from_numpy(lg).to(DEV), k, qgu, qd, I)
    torch.cuda.synchronize()
    ref, rr = oracle.moe_layer(to_f32(x), lg, k, oracle.quantize(fmt, to_f32(wgu)),
                               oracle.quantize(fmt, to_f32(wd)), I)
    assert np.array_equal(r.ids.cpu().numpy(), rr.ids)
    _check_layer(out, ref, f"moe layer {fmt} {layout}")


def test_moe_layer_expert_shape():
    """The MoE workload's per-expert shapes (W_gate/W_up 2048 x 7168, W_down
    7168 x 2048, MXFP4, tiled) with 8 experts, 64 tokens, top-2; 16 tokens
    checked against the oracle."""
    E, T, k = 8, 64, 2
    wl = workloads.moe_layer(experts=E, tokens=T, topk=k)
    I, K = wl.meta["I"], wl.meta["K"]
    log("moe layer expert shape: generating weights")
    experts = [wl.meta["expert"](e) for e in range(E)]
    wgu = torch.cat([g for g, _ in experts])
    wd = torch.cat([d for _, d in experts])
    x = wl.tensors["x"][:T]
    lg = wl.meta["logits"][:T, :E].copy()
    qgu = q4.quantize(wgu.to(DEV), "mxfp4", layout="tiled")
    qd = q4.quantize(wd.to(DEV), "mxfp4", layout="tiled")
    out, r = q4.moe_layer(x.to(DEV), torch.from_numpy(lg).to(DEV), k, qgu, qd, I)
    torch.cuda.synchronize()
    tokens = list(range(0, T, 4))
    log("moe layer expert shape: oracle")
    ref, rr = oracle.moe_layer(to_f32(x), lg, k, oracle.quantize("mxfp4", to_f32(wgu)),
                               oracle.quantize("mxfp4", to_f32(wd)), I, tokens=tokens)
    assert np.array_equal(r.ids.cpu().numpy(), rr.ids)
    _check_layer(out[tokens], ref, "moe layer 2048x7168")


@pytest.mark.parametrize("fmt", ("mxfp4", "int4", "nvfp4", "int4_zp"))
@pytest.mark.parametrize("E,I,K,T,k", [(8, 512, 1024, 37, 2), (4, 272, 512, 300, 2)])
def test_grouped_gemm_swiglu(fmt, E, I, K, T, k):
    """The fused gate/up + SwiGLU epilogue against the oracle's grouped GEMM
    followed by SwiGLU; bad gather rows give zero rows."""
    log("grouped gemm swiglu", fmt, E, I, K, T, k)
    wgu = workloads.matrix(f"tmoe/fw{E}x{I}x{K}", E * 2 * I, K, 0.03, seed=90)
    a = workloads.matrix(f"tmoe/fa{T}x{K}", T, K, 1.0, seed=91)
    lg = _logits(T, E, seed=92)
    rr = oracle.moe_route(lg, k)
    gather = rr.gather.copy()
    gather[5] = -1
    gather[7] = T + 3
    qw = q4.quantize(q4.interleave_gate_up(wgu, E, I).to(DEV), fmt, layout="tiled")
    P = len(gather)
    H = torch.full((P, I + 8), float("nan"), dtype=torch.bfloat16, device=DEV)
    q4.q4_grouped_gemm_swiglu(a.to(DEV), torch.from_numpy(gather).to(DEV), torch.from_numpy(rr.offsets).to(DEV),
                              qw, I, H[:, :I])
    torch.cuda.synchronize()
    Hc = H.cpu()
    assert torch.isnan(Hc[:, I:]).all()
    got = to_f32(Hc[:, :I]).astype(np.float64)
    qr = oracle.quantize(fmt, to_f32(wgu))
    gu = oracle.grouped_gemm(to_f32(a), np.clip(gather, 0, T - 1), rr.offsets, qr, 2 * I)
    ref = oracle.swiglu(gu, I)
    bad_rows = [5, 7]
    ref[bad_rows] = 0.0
    assert np.all(got[bad_rows] == 0.0)
    # error bound: bf16 output rounding plus the propagated error of the two sums
    af = np.abs(to_f32(a).astype(np.float64))
    wd = np.abs(oracle.dequant(qr).astype(np.float64))
    S = np.zeros((P, 2 * I))
    for e in range(E):
        lo, hi = rr.offsets[e], rr.offsets[e + 1]
        S[lo:hi] = af[np.clip(gather[lo:hi], 0, T - 1)] @ wd[e * 2 * I:(e + 1) * 2 * I].T
    c = 2.0 ** -16 if fmt == "mxfp4" else 2.0 ** -8
    g, u = gu[:, :I], gu[:, I:]
    bound = 2.0 ** -8 * np.abs(ref) + 1.1 * c * (S[:, :I] * np.abs(u) + np.abs(g) * S[:, I:]) + c * c * S[:, :I] * S[:, I:] + 1e-30
    bound[bad_rows] = 0.0
    bad = np.argwhere(np.abs(got - ref) > bound)
    assert bad.size == 0, [(int(i), int(j), got[i, j], ref[i, j]) for i, j in bad[:5]]


@pytest.mark.parametrize("fmt", ("mxfp4", "nvfp4"))
def test_moe_layer_fused(fmt):
    E, I, K, T, k = 8, 512, 1024, 37, 2
    log("moe layer fused", fmt)
    wgu = workloads.matrix("tmoe/wgu", E * 2 * I, K, 0.03, seed=86)
    wd = workloads.matrix("tmoe/wd", E * K, I, 0.03, seed=87)
    x = workloads.matrix("tmoe/x", T, K, 1.0, seed=88)
    lg = _logits(T, E, seed=89)
    qgu = q4.quantize(q4.interleave_gate_up(wgu, E, I).to(DEV), fmt, layout="tiled")
    qd = q4.quantize(wd.to(DEV), fmt, layout="tiled")
    out, r = q4.moe_layer(x.to(DEV), torch.from_numpy(lg).to(DEV), k, qgu, qd, I, fused=True)
    torch.cuda.synchronize()
    ref, rr = oracle.moe_layer(to_f32(x), lg, k, oracle.quantize(fmt, to_f32(wgu)),
                               oracle.quantize(fmt, to_f32(wd)), I)
    _check_layer(out, ref, f"moe layer fused {fmt}")


@pytest.mark.parametrize("E,k", [(64, 8), (16, 4), (70, 3)])
def test_route_nan_logits_fill_every_slot(E, k):
    """NaN router logits have no order in the pages, but the routing stays a
    routing: every one of the token's k slots names a distinct expert (the
    outputs start filled with -1, through the C ABI), the dispatch order is a
    permutation, and tokens without NaN route exactly as the oracle does."""
    log("route nan", E, k)
    T = 12
    lg = _logits(T, E, seed=83)
    lg[0, 3] = np.nan
    lg[1, :] = np.nan                                   # all NaN
    lg[2, 5] = -np.float32(np.nan)                       # sign bit set
    lg[4, : min(E, 6)] = np.nan
    d = torch.from_numpy(lg).to(DEV)
    ids = torch.full((T, k), -1, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), -1.0, dtype=torch.float32, device=DEV)
    off = torch.full((E + 1,), -1, dtype=torch.int32, device=DEV)
    gather = torch.full((T * k,), -1, dtype=torch.int32, device=DEV)
    inv = torch.full((T, k), -1, dtype=torch.int32, device=DEV)
    rc = q4.lib().q4_moe_route(q4._ptr(d), E, T, E, k, q4._ptr(ids), q4._ptr(w), q4._ptr(off), q4._ptr(gather),
                               q4._ptr(inv), None)
    torch.cuda.synchronize()
    assert rc == 0
    ids_h, off_h, g_h, inv_h = ids.cpu().numpy(), off.cpu().numpy(), gather.cpu().numpy(), inv.cpu().numpy()
    for t in range(T):
        assert len(set(ids_h[t])) == k and ids_h[t].min() >= 0 and ids_h[t].max() < E, (t, ids_h[t])
    assert off_h[0] == 0 and off_h[E] == T * k and (np.diff(off_h) >= 0).all()
    assert sorted(inv_h.reshape(-1)) == list(range(T * k))
    for i, pos in enumerate(inv_h.reshape(-1)):
        assert g_h[pos] == i // k
        e = ids_h.reshape(-1)[i]
        assert off_h[e] <= pos < off_h[e + 1]
    clean = [t for t in range(T) if not np.isnan(lg[t]).any()]
    ref = oracle.moe_route(np.ascontiguousarray(lg[clean]), k)
    assert np.array_equal(ids_h[clean], ref.ids)
    assert np.allclose(w.cpu().numpy()[clean].astype(np.float64), ref.weights, rtol=2e-6, atol=1e-30)


def test_full_gate_up_swiglu():
    """The fused gate/up + SwiGLU grouped GEMM at the MoE layer the benchmark
    times (64 experts of 2 x 2048 x 7168, MXFP4 tiled, 256 tokens, top-8, the
    MoE workload's x and router logits): 24 sampled routed rows, all 2048
    outputs each, against the oracle's grouped GEMM and SwiGLU for their
    experts.  The weights are drawn as the benchmark draws them (torch's
    generator on the GPU, N(0, 0.02^2)) and the sampled experts' bf16 rows
    copied to the host for the oracle."""
    E, I, K, T, k = 64, 2048, 7168, 256, 8
    log("full gate/up swiglu: weights")
    g = torch.Generator(device=DEV).manual_seed(5)
    wgu = (torch.randn((E * 2 * I, K), generator=g, device=DEV) * 0.02).bfloat16()
    qw = q4.quantize(q4.interleave_gate_up(wgu, E, I), "mxfp4", layout="tiled")
    x = workloads.matrix("moe/A", T, K, 1.0, 0)
    lg = workloads.normal_f32("moe/logits", T * E, 0).reshape(T, E)
    rr = oracle.moe_route(lg, k)
    P = T * k
    H = torch.empty((P, I), dtype=torch.bfloat16, device=DEV)
    q4.q4_grouped_gemm_swiglu(x.to(DEV), torch.from_numpy(rr.gather).to(DEV),
                              torch.from_numpy(rr.offsets).to(DEV), qw, I, H)
    torch.cuda.synchronize()
    pick = np.unique(np.concatenate([[0, P - 1], np.random.default_rng(7).choice(P, 22, replace=False)]))
    got = to_f32(H[torch.from_numpy(pick).to(DEV)].cpu()).astype(np.float64)
    xa = to_f32(x)
    expert_of = np.searchsorted(rr.offsets, pick, side="right") - 1
    for e in np.unique(expert_of):
        log("full gate/up swiglu: oracle, expert", int(e))
        sel = np.nonzero(expert_of == e)[0]
        a = xa[rr.gather[pick[sel]]]
        wd = oracle.dequant(oracle.quantize("mxfp4", to_f32(wgu[e * 2 * I:(e + 1) * 2 * I].cpu())))
        gu = oracle.matmul_f64(a, wd)
        ref = oracle.swiglu(gu, I)
        S = np.abs(a.astype(np.float64)) @ np.abs(wd.astype(np.float64)).T
        c = 2.0 ** -16
        gg, uu = gu[:, :I], gu[:, I:]
        bound = (2.0 ** -8 * np.abs(ref) + 1.1 * c * (S[:, :I] * np.abs(uu) + np.abs(gg) * S[:, I:])
                 + c * c * S[:, :I] * S[:, I:] + 1e-30)
        err = np.abs(got[sel] - ref)
        bad = np.argwhere(err > bound)
        assert bad.size == 0, (int(e), [(int(i), int(j), got[sel][i, j], ref[i, j]) for i, j in bad[:5]])
