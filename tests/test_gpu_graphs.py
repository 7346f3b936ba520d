"""The library's calls inside a captured HIP graph: every replay gives the
bytes the eager call gave.  Between replays the outputs are overwritten and
other eager work runs on the same buffers' neighbours, with a
synchronization, so that a replay that kept state from an earlier one (a
counter or word not reset inside the graph, a memset node replayed wrongly)
shows as a difference.  The library records kernels only (the NVFP4
quantizer resets its tensor-amax word with a kernel, not a memset)."""
import pytest
import torch

import w4_gemm_amd as q4
from q4_helpers import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


def _bytes(t: torch.Tensor) -> bytes:
    return t.detach().contiguous().cpu().view(torch.uint8).numpy().tobytes()


def _outs_bytes(outs):
    return [_bytes(t) for t in outs]


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    return g, outs


def _check_replays(fn, scribble, other):
    """fn() runs the call and returns its output tensors; scribble(outs)
    overwrites them; other() is unrelated eager work."""
    ref = _outs_bytes(fn())
    torch.cuda.synchronize()
    g, outs = _capture(fn)
    for rep in range(REPLAYS):
        scribble(outs)
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outs_bytes(outs)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert a == b, f"replay {rep}: output {i} differs from the eager call"


def _q4_outs(q):
    return [q.codes, q.scales] + ([q.global_scale] if q.global_scale is not None else [])


def _scribble(outs):
    for t in outs:
        if t.dtype == torch.float32:
            t.fill_(-3.0)
        else:
            t.view(torch.uint8).fill_(0xA5)


def _rand(shape, seed, scale=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(*shape, device=DEV, generator=g) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("fmt,layout", [("nvfp4", "tiled"), ("nvfp4", "rows"), ("mxfp4", "tiled"),
                                        ("int4_zp", "tiled")])
def test_graph_quantize(fmt, layout):
    log("graph quantize", fmt, layout)
    w = _rand((80, 1024), 1, 0.02)
    w2 = _rand((80, 1024), 2, 0.5)
    dst = q4.empty_q4(fmt, 80, 1024, device=DEV, layout=layout)
    other_dst = q4.empty_q4(fmt, 80, 1024, device=DEV, layout=layout)

    def fn():
        q4.q4_quantize(w, dst)
        return _q4_outs(dst)

    # the unrelated work quantizes a tensor with a larger amax (a stale
    # tensor-amax word would carry it into the replay)
    _check_replays(fn, _scribble, lambda: q4.q4_quantize(w2, other_dst))


def test_graph_gemv_and_gemm():
    log("graph gemv, gemm")
    N, K = 272, 1024
    W = _rand((N, K), 3, 0.02)
    qm = q4.quantize(W, "mxfp4", layout="tiled")
    qn = q4.quantize(W, "nvfp4", layout="tiled")
    x = _rand((16, K), 4)
    A = _rand((96, K), 5)
    qa = q4.quantize(A, "mxfp4", layout="tiled")
    y = torch.empty(16, N, device=DEV, dtype=torch.bfloat16)
    C1 = torch.empty(96, N, device=DEV, dtype=torch.bfloat16)
    C2 = torch.empty_like(C1)
    gsq = torch.tensor([0.01], device=DEV, dtype=torch.float32)
    Cq = q4.empty_q4("nvfp4", 96, N - 16, device=DEV, layout="rows")
    Wq = q4.quantize(W[: N - 16].contiguous(), "mxfp4", layout="tiled")

    def fn():
        q4.q4_gemv(qm, x, y)
        q4.q4_gemm(A, qn, C1)
        q4.q4_gemm(qa, qm, C2)
        q4.q4_gemm_quantized(A, Wq, Cq, nv_global_in=gsq)
        return [y, C1, C2] + _q4_outs(Cq)

    _check_replays(fn, _scribble, lambda: q4.q4_gemm(A, qm, C1))


@pytest.mark.parametrize("fused", (False, True))
def test_graph_moe_layer(fused):
    log("graph moe layer, fused", fused)
    T, E, k, K, inter = 40, 8, 2, 512, 512
    x = _rand((T, K), 6)
    logits = torch.randn(T, E, device=DEV, generator=torch.Generator(device=DEV).manual_seed(7))
    wgu = _rand((E * 2 * inter, K), 8, 0.02)
    if fused:
        wgu = q4.interleave_gate_up(wgu, E, inter)
    W_gu = q4.quantize(wgu, "mxfp4", layout="tiled")
    W_down = q4.quantize(_rand((E * K, inter), 10, 0.02), "mxfp4", layout="tiled")

    def fn():
        out, r = q4.moe_layer(x, logits, k, W_gu, W_down, inter, fused=fused)
        return [out, r.ids, r.weights, r.offsets, r.gather, r.inv]

    _check_replays(fn, _scribble, lambda: q4.q4_moe_route(logits.flip(0).contiguous(), k))


def test_graph_relayout():
    log("graph relayout")
    w = _rand((50, 1024), 11, 0.02)
    src = q4.quantize(w, "nvfp4", layout="rows")
    dst = q4.empty_q4("nvfp4", 50, 1024, device=DEV, layout="tiled")

    def fn():
        q4.q4_relayout(src, dst)
        return _q4_outs(dst)

    _check_replays(fn, _scribble, lambda: q4.q4_quantize(w, src))


def test_graph_w4a8_w4a4nv_dequant():
    """The other GEMM chains (activation quantize, then the GEMM) and the
    dequantizer: W4A8 (per-token FP8 activations x INT4 weights), W4A4 NVFP4
    (the activation's tensor amax recomputed inside the graph), and MXFP4 /
    NVFP4 weights dequantized to bf16 and fp32."""
    log("graph w4a8, w4a4 nvfp4, dequant")
    M, N, K = 96, 272, 1024
    A = _rand((M, K), 12)
    A2 = _rand((M, K), 13, 4.0)
    W = _rand((N, K), 14, 0.02)
    qw8 = q4.quantize(W, "int4", layout="tiled")
    qwn = q4.quantize(W, "nvfp4", layout="tiled")
    qwm = q4.quantize(W, "mxfp4", layout="tiled")
    qwr = q4.quantize(W, "nvfp4", layout="rows")
    qa8 = q4.empty_q4("fp8_row", M, K, device=DEV, layout="tiled")
    qan = q4.empty_q4("nvfp4", M, K, device=DEV, layout="tiled")
    C8 = torch.empty(M, N, device=DEV, dtype=torch.bfloat16)
    Cn = torch.empty_like(C8)
    D16 = torch.empty(N, K, device=DEV, dtype=torch.bfloat16)
    D32 = torch.empty(N, K, device=DEV, dtype=torch.float32)
    other_a8 = q4.empty_q4("fp8_row", M, K, device=DEV, layout="tiled")
    other_an = q4.empty_q4("nvfp4", M, K, device=DEV, layout="tiled")

    def fn():
        q4.q4_quantize(A, qa8)
        q4.q4_gemm(qa8, qw8, C8)
        q4.q4_quantize(A, qan)
        q4.q4_gemm(qan, qwn, Cn)
        q4.q4_dequant(qwm, D16)
        q4.q4_dequant(qwr, D32)
        return [C8, Cn, D16, D32] + _q4_outs(qa8) + _q4_outs(qan)

    def other():
        # a larger-amax tensor through the same quantizers and GEMMs
        q4.q4_quantize(A2, other_a8)
        q4.q4_quantize(A2, other_an)
        q4.q4_gemm(other_an, qwn, Cn)

    _check_replays(fn, _scribble, other)
