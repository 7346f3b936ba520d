"""The Python binding rejects bad arguments before any library call.

A wrong tensor handed to the C ABI would reach a kernel as a raw pointer:
a host address, a buffer too small for the rows written, a dtype read as
another.  Each wrapper in w4_gemm_amd checks dtypes, shapes, strides and
buffer sizes, then that every tensor is on the GPU, and raises ValueError
first.  Here (no GPU) every bad case must raise, and no call may get past
the checks: the library handle is replaced by a guard that lets only the
host-side size query through.
"""
import pytest
import torch

import w4_gemm_amd as q4

BF16, F32, I32 = torch.bfloat16, torch.float32, torch.int32


class _Guard:
    """Stands in for libq4.so: q4_sizes (host arithmetic only) passes
    through, any other call fails the test."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in ("q4_sizes", "q4_status_string", "q4_last_hip_error"):
            return getattr(self._real, name)
        raise AssertionError(f"{name} was called with invalid arguments")


@pytest.fixture(autouse=True)
def guard(monkeypatch):
    real = q4.lib()
    monkeypatch.setattr(q4, "_LIB", _Guard(real))
    yield


def _w(fmt="mxfp4", rows=64, cols=512, layout=q4.LAYOUT_ROWS):
    return q4.empty_q4(fmt, rows, cols, device="cpu", layout=layout)


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_gemv_rejects():
    W = _w()
    x = torch.zeros(4, 512, dtype=BF16)
    y = torch.zeros(4, 64, dtype=BF16)
    _raises("x must be torch.bfloat16", q4.q4_gemv, W, x.float(), y)
    _raises("x must have 512 columns", q4.q4_gemv, W, torch.zeros(4, 256, dtype=BF16), y)
    _raises("x must be 2-D", q4.q4_gemv, W, torch.zeros(512, dtype=BF16), y)
    _raises("y must be at least 4 x 64", q4.q4_gemv, W, x, y[:2])
    _raises("y must be at least 4 x 64", q4.q4_gemv, W, x, y[:, :32])
    _raises("y must be torch.bfloat16", q4.q4_gemv, W, x, y.float())
    _raises("x must have unit column stride", q4.q4_gemv, W, torch.zeros(512, 4, dtype=BF16).t(), y)
    _raises("y must have unit column stride", q4.q4_gemv, W, x, torch.zeros(64, 4, dtype=BF16).t())
    bad = _w()
    bad.codes = bad.codes[:10]
    _raises("W.codes must be contiguous and hold", q4.q4_gemv, bad, x, y)
    bad = _w()
    bad.scales = bad.scales[:, ::2]
    _raises("W.scales must be contiguous", q4.q4_gemv, bad, x, y)
    nv = _w("nvfp4")
    nv.global_scale = None
    _raises("global_scale is required", q4.q4_gemv, nv, x, y)
    # every shape right, but host tensors
    _raises("must be a GPU tensor", q4.q4_gemv, W, x, y)


def test_gemm_rejects():
    W = _w()
    A = torch.zeros(32, 512, dtype=BF16)
    C = torch.zeros(32, 64, dtype=BF16)
    _raises("A must have 512 columns", q4.q4_gemm, torch.zeros(32, 1024, dtype=BF16), W, C)
    _raises("A must be torch.bfloat16", q4.q4_gemm, A.float(), W, C)
    _raises("C must be at least 32 x 64", q4.q4_gemm, A, W, C[:31])
    _raises("C must be torch.bfloat16", q4.q4_gemm, A, W, C.float())
    Aq = _w(rows=32, cols=1024)
    _raises("A has 1024 columns", q4.q4_gemm, Aq, W, C)
    Aq = _w(rows=40)
    _raises("C must be at least 40 x 64", q4.q4_gemm, Aq, W, C)
    _raises("must be a GPU tensor", q4.q4_gemm, A, W, C)
    _raises("must be a GPU tensor", q4.q4_gemm, _w(rows=32), W, C)


def test_grouped_rejects():
    E, N, K, T = 4, 32, 512, 8
    W = _w(rows=E * N, cols=K, layout=q4.LAYOUT_TILED)
    A = torch.zeros(T, K, dtype=BF16)
    gather = torch.zeros(16, dtype=I32)
    offsets = torch.zeros(E + 1, dtype=I32)
    C = torch.zeros(16, N, dtype=BF16)
    _raises("offsets must be a torch.int32", q4.q4_grouped_gemm, A, gather, offsets.long(), W, N, C)
    _raises("gather must be a torch.int32", q4.q4_grouped_gemm, A, gather.long(), offsets, W, N, C)
    _raises("not experts", q4.q4_grouped_gemm, A, gather, offsets[:3], W, N, C)
    _raises("not experts", q4.q4_grouped_gemm, A, gather, offsets, W, 16, C)
    _raises("C must be at least 16 x 32", q4.q4_grouped_gemm, A, gather, offsets, W, N, C[:15])
    _raises("A must have 512 columns", q4.q4_grouped_gemm, A[:, :256], gather, offsets, W, N, C)
    _raises("gather must be contiguous", q4.q4_grouped_gemm, A, torch.zeros(32, dtype=I32)[::2],
            offsets, W, N, C)
    _raises("must be a GPU tensor", q4.q4_grouped_gemm, A, gather, offsets, W, N, C)
    # the fused gate/up + SwiGLU variant
    I = 16
    Wgu = _w(rows=E * 2 * I, cols=K, layout=q4.LAYOUT_TILED)
    H = torch.zeros(16, I, dtype=BF16)
    _raises("not experts", q4.q4_grouped_gemm_swiglu, A, gather, offsets, Wgu, 32, H)
    _raises("H must be at least 16 x 16", q4.q4_grouped_gemm_swiglu, A, gather, offsets, Wgu, I, H[:8])
    _raises("must be a GPU tensor", q4.q4_grouped_gemm_swiglu, A, gather, offsets, Wgu, I, H)


def test_quantize_and_dequant_reject():
    dst = _w(rows=16, cols=512)
    src = torch.zeros(16, 512, dtype=BF16)
    _raises("src must be at least 16 x 512", q4.q4_quantize, src[:8], dst)
    _raises("src must be at least 16 x 512", q4.q4_quantize, src[:, :256], dst)
    _raises("src must be torch.bfloat16", q4.q4_quantize, src.float(), dst)
    nv = _w("nvfp4", rows=16, cols=512)
    _raises("nv_global_in must be a torch.float32", q4.q4_quantize, src, nv, torch.zeros(1, dtype=torch.float64))
    _raises("must be a GPU tensor", q4.q4_quantize, src, dst)
    out = torch.zeros(16, 512, dtype=F32)
    _raises("dst must be at least 16 x 512", q4.q4_dequant, dst, out[:, :500])
    _raises("dst must be bf16 or float32", q4.q4_dequant, dst, out.double())
    _raises("must be a GPU tensor", q4.q4_dequant, dst, out)


def test_moe_helpers_reject():
    T, k, E, N, I = 4, 2, 8, 64, 32
    _raises("logits must be torch.float32", q4.q4_moe_route, torch.zeros(T, E, dtype=BF16), k)
    _raises("must be a GPU tensor", q4.q4_moe_route, torch.zeros(T, E), k)
    gu = torch.zeros(T * k, 2 * I, dtype=BF16)
    _raises("gu must be at least 0 x 64", q4.q4_swiglu, gu[:, :I], I)
    _raises("h must be at least 8 x 32", q4.q4_swiglu, gu, I, torch.zeros(4, I, dtype=BF16))
    _raises("must be a GPU tensor", q4.q4_swiglu, gu, I, torch.zeros(T * k, I, dtype=BF16))
    r = q4.Routing(torch.zeros(T, k, dtype=I32), torch.zeros(T, k), torch.zeros(E + 1, dtype=I32),
                   torch.zeros(T * k, dtype=I32), torch.zeros(T, k, dtype=I32))
    y = torch.zeros(T * k, N, dtype=BF16)
    _raises("y must be at least 8 x 0", q4.q4_moe_combine, y[:5], r)
    _raises("out must be at least 4 x 64", q4.q4_moe_combine, y, r, torch.zeros(T, 32, dtype=BF16))
    bad = q4.Routing(r.ids, r.weights.double(), r.offsets, r.gather, r.inv)
    _raises("r.weights must be a torch.float32", q4.q4_moe_combine, y, bad)
    _raises("must be a GPU tensor", q4.q4_moe_combine, y, r, torch.zeros(T, N, dtype=BF16))


def test_relayout_rejects():
    a = q4.empty_q4("mxfp4", 32, 512, device="cpu")
    b = q4.empty_q4("mxfp4", 32, 512, device="cpu", layout="tiled")
    _raises("same format and shape", q4.q4_relayout, a, q4.empty_q4("nvfp4", 32, 512, device="cpu", layout="tiled"))
    _raises("same format and shape", q4.q4_relayout, a, q4.empty_q4("mxfp4", 48, 512, device="cpu", layout="tiled"))
    _raises("must be a Q4Tensor", q4.q4_relayout, a, b.codes)
    _raises("must be a GPU tensor", q4.q4_relayout, a, b)


def test_mfma_probe_rejects():
    sink = torch.zeros(1, dtype=I32)
    _raises("kind must be one of", q4.q4_mfma_probe, "int8", 16, sink)
    _raises("iters must be an int", q4.q4_mfma_probe, "fp4", -1, sink)
    _raises("iters must be an int", q4.q4_mfma_probe, "fp4", 1.5, sink)
    _raises("sink must be a torch.int32", q4.q4_mfma_probe, "fp4", 16, sink.float())
    _raises("must be a GPU tensor", q4.q4_mfma_probe, "bf16", 16, sink)
    _raises("sink must be contiguous with at least 16384 entries", q4.q4_mfma_probe, "fp4_mix", 16, sink)
    _raises("sink must be contiguous with at least 16384 entries", q4.q4_mfma_probe, "fp4_copy", 16, sink)
    _raises("sink must be contiguous with at least 16384 entries", q4.q4_mfma_probe, "bf16_mix", 16, sink)
