"""The C ABI of libq4.so on the host: it loads without a GPU, exports every
function include/q4.h declares, and rejects bad arguments with the right
status before any HIP call (no call here reaches a launch)."""
import ctypes
import os
import re

import pytest

import w4_gemm_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4.h")

OK, NULL, SHAPE, ALIGN, FMT = 0, -1, -2, -3, -4

# Fake device addresses: never dereferenced, since every call below fails
# validation (or is a no-op) before reaching a kernel.
A16 = 0x7F0000000000
A_ODD = A16 + 2


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(q4_\w+)\s*\(", text, re.M)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("q4_quantize", "q4_dequant", "q4_gemv", "q4_gemm", "q4_grouped_gemm",
              "q4_moe_route", "q4_swiglu", "q4_moe_combine"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = q4.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert q4.q4_version() >= 100


def test_status_strings():
    L = q4.lib()
    for st in (0, -1, -2, -3, -4, -6):
        assert L.q4_status_string(st)
    assert L.q4_status_string(12345) == b"unknown status"
    assert L.q4_last_hip_error() == 0


@pytest.mark.parametrize("fmt,cols,codes,scales", [
    (q4.INT4_G128, 1024, 512, 16), (q4.MXFP4, 1024, 512, 32), (q4.NVFP4, 1024, 512, 64),
    (q4.INT4_ZP, 1024, 512, 32),
])
def test_sizes(fmt, cols, codes, scales):
    assert q4.q4_sizes(fmt, 1, cols) == (codes, scales)
    assert q4.q4_sizes(fmt, 28672, 8192)[0] == 28672 * 4096
    assert q4.q4_sizes(fmt, 0, cols) == (0, 0)
    # tiled: whole 16-row tiles, the same bytes per stored row
    assert q4.q4_sizes(fmt, 1, cols, "tiled") == (16 * codes, 16 * scales)
    assert q4.q4_sizes(fmt, 32, cols, "tiled") == (32 * codes, 32 * scales)


def test_sizes_rejects():
    L = q4.lib()
    assert L.q4_sizes(7, 0, 1, 128, None, None) == FMT
    assert L.q4_sizes(q4.MXFP4, 5, 1, 128, None, None) == FMT
    assert L.q4_sizes(q4.MXFP4, 0, 1, 48, None, None) == SHAPE
    assert L.q4_sizes(q4.INT4_G128, 0, 1, 64, None, None) == SHAPE
    assert L.q4_sizes(q4.MXFP4, 0, -1, 64, None, None) == SHAPE
    assert L.q4_sizes(q4.MXFP4, 1, 1, 256, None, None) == SHAPE   # tiled: cols % 512


def desc(fmt=q4.MXFP4, rows=64, cols=256, codes=A16, scales=A16, gs=None, layout=0):
    return q4._Q4TensorC(fmt, layout, rows, cols, codes, scales, gs)


def call_quantize(src, ld, d, gs_in=None):
    return q4.lib().q4_quantize(src, ld, ctypes.byref(d), gs_in, None)


def test_quantize_validation():
    L = q4.lib()
    assert L.q4_quantize(A16, 256, None, None, None) == NULL
    assert call_quantize(None, 256, desc()) == NULL
    assert call_quantize(A16, 256, desc(fmt=9)) == FMT
    assert call_quantize(A16, 256, desc(layout=2)) == FMT
    assert call_quantize(A16, 256, desc(layout=1)) == SHAPE       # tiled needs cols % 512
    assert call_quantize(A16, 512, desc(layout=1, cols=512, rows=0)) == OK
    assert call_quantize(A16, 256, desc(cols=48)) == SHAPE
    assert call_quantize(A16, 256, desc(rows=-1)) == SHAPE
    assert call_quantize(A16, 128, desc()) == SHAPE              # ld < cols
    assert call_quantize(A16, 260, desc()) == ALIGN              # ld not a multiple of 8
    assert call_quantize(A_ODD, 256, desc()) == ALIGN
    assert call_quantize(A16, 256, desc(codes=A16 + 4)) == ALIGN
    assert call_quantize(A16, 256, desc(codes=None)) == NULL
    assert call_quantize(A16, 256, desc(fmt=q4.NVFP4)) == NULL   # NVFP4 needs global_scale
    assert call_quantize(A16, 256, desc(gs=A16)) == FMT          # only NVFP4 takes one
    assert call_quantize(A16, 256, desc(), gs_in=A16) == FMT
    assert call_quantize(A16, 256, desc(rows=0)) == OK           # empty: no launch


def test_dequant_validation():
    L = q4.lib()
    d = desc()
    assert L.q4_dequant(ctypes.byref(d), A16, 2, 256, None) == FMT
    assert L.q4_dequant(ctypes.byref(d), None, 0, 256, None) == NULL
    assert L.q4_dequant(ctypes.byref(d), A16, 0, 100, None) == SHAPE
    assert L.q4_dequant(ctypes.byref(d), A16, 1, 258, None) == ALIGN
    assert L.q4_dequant(ctypes.byref(desc(rows=0)), None, 0, 256, None) == OK


def test_gemv_validation():
    L = q4.lib()
    d = desc(rows=1024, cols=1024)
    assert L.q4_gemv(ctypes.byref(d), A16, 17, 1024, A16, 1024, None) == SHAPE
    assert L.q4_gemv(ctypes.byref(d), A16, -1, 1024, A16, 1024, None) == SHAPE
    assert L.q4_gemv(ctypes.byref(desc(rows=8, cols=96)), A16, 1, 96, A16, 8, None) == SHAPE
    assert L.q4_gemv(ctypes.byref(d), None, 1, 1024, A16, 1024, None) == NULL
    assert L.q4_gemv(ctypes.byref(d), A16, 1, 1024, None, 1024, None) == NULL
    assert L.q4_gemv(ctypes.byref(d), A16, 2, 1000, A16, 1024, None) == SHAPE
    assert L.q4_gemv(ctypes.byref(d), A16, 2, 1024, A16, 1000, None) == SHAPE
    assert L.q4_gemv(ctypes.byref(d), A_ODD, 1, 1024, A16, 1024, None) == ALIGN
    assert L.q4_gemv(ctypes.byref(d), A16, 0, 1024, A16, 1024, None) == OK


def test_gemm_validation():
    L = q4.lib()
    w = desc(rows=512, cols=512)
    a = desc(rows=64, cols=512)
    nv = desc(fmt=q4.NVFP4, rows=64, cols=512, gs=A16)
    assert L.q4_gemm(64, A16, 512, ctypes.byref(a), ctypes.byref(w), A16, 512, None) == FMT
    assert L.q4_gemm(64, None, 512, None, ctypes.byref(w), A16, 512, None) == NULL
    assert L.q4_gemm(64, None, 0, ctypes.byref(nv), ctypes.byref(w), A16, 512, None) == FMT
    # W4A4 takes both operands in one FP4 format: NVFP4 x NVFP4 is accepted
    nvw = desc(fmt=q4.NVFP4, rows=512, cols=512, gs=A16)
    assert L.q4_gemm(64, None, 0, ctypes.byref(a), ctypes.byref(nvw), A16, 512, None) == FMT
    assert L.q4_gemm(64, None, 0, ctypes.byref(nv), ctypes.byref(desc(fmt=q4.INT4_G128, rows=512, cols=512)),
                     A16, 512, None) == FMT
    assert L.q4_gemm(32, None, 0, ctypes.byref(nv), ctypes.byref(nvw), A16, 512, None) == SHAPE
    assert L.q4_gemm(64, None, 0, ctypes.byref(nv), ctypes.byref(desc(fmt=q4.NVFP4, rows=512, cols=512)),
                     A16, 512, None) == NULL                      # an NVFP4 weight needs its global scale
    assert L.q4_gemm(0, None, 0, ctypes.byref(desc(fmt=q4.NVFP4, rows=0, cols=512, gs=A16)),
                     ctypes.byref(nvw), A16, 512, None) == OK
    assert L.q4_gemm(32, None, 0, ctypes.byref(a), ctypes.byref(w), A16, 512, None) == SHAPE
    assert L.q4_gemm(64, A16, 512, None, ctypes.byref(desc(rows=512, cols=96)), A16, 512,
                     None) == SHAPE
    assert L.q4_gemm(64, A16, 500, None, ctypes.byref(w), A16, 512, None) == SHAPE
    assert L.q4_gemm(64, A16, 512, None, ctypes.byref(w), A16, 500, None) == SHAPE
    assert L.q4_gemm(-1, A16, 512, None, ctypes.byref(w), A16, 512, None) == SHAPE
    assert L.q4_gemm(0, A16, 512, None, ctypes.byref(w), A16, 512, None) == OK


def test_fp8_rows_sizes_and_formats():
    assert q4.q4_sizes(q4.FP8_ROW, 3, 1024) == (3 * 1024, 3 * 4)
    assert q4.q4_sizes(q4.FP8_ROW, 3, 1024, "tiled") == (16 * 1024, 3 * 4)
    with pytest.raises(q4.Q4Error):
        q4.q4_sizes(q4.FP8_ROW, 3, 1000)
    L = q4.lib()
    w4 = desc(fmt=q4.INT4_G128, rows=512, cols=512)
    mx = desc(fmt=q4.MXFP4, rows=512, cols=512)
    a8 = desc(fmt=q4.FP8_ROW, rows=64, cols=512)
    # W4A8 needs an INT4 weight; an FP8 tensor is never a weight
    assert L.q4_gemm(64, None, 0, ctypes.byref(a8), ctypes.byref(mx), A16, 512, None) == FMT
    assert L.q4_gemm(64, None, 0, ctypes.byref(a8), ctypes.byref(a8), A16, 512, None) == FMT
    assert L.q4_gemm(64, A16, 512, None, ctypes.byref(a8), A16, 512, None) == FMT
    assert L.q4_gemm(32, None, 0, ctypes.byref(a8), ctypes.byref(w4), A16, 512, None) == SHAPE
    assert L.q4_gemm(0, None, 0, ctypes.byref(desc(fmt=q4.FP8_ROW, rows=0, cols=512)),
                     ctypes.byref(w4), A16, 512, None) == OK
    assert L.q4_gemv(ctypes.byref(a8), A16, 1, 512, A16, 512, None) == FMT
    assert L.q4_quantize(A16, 512, ctypes.byref(a8), A16, None) == FMT   # no global scale input


def test_grouped_validation():
    L = q4.lib()
    w = desc(rows=8 * 128, cols=512)
    ok_args = dict(A=A16, lda=512, T=16, gather=A16, off=A16, E=8, P=32, N=128, C=A16, ldc=128)

    def call(**kw):
        a = dict(ok_args, **kw)
        return L.q4_grouped_gemm(a["A"], a["lda"], a["T"], a["gather"], a["off"], a["E"], a["P"],
                                 ctypes.byref(kw.get("W", w)), a["N"], a["C"], a["ldc"], None)

    assert call(N=100) == SHAPE                  # W rows != E*N
    assert call(E=-1) == SHAPE
    assert call(gather=None) == SHAPE          # identity gather needs T >= P
    assert call(off=None) == NULL
    assert call(gather=A16 + 2) == ALIGN
    assert call(lda=500) == SHAPE
    assert call(ldc=100) == SHAPE
    assert call(P=0) == OK
    assert call(W=desc(rows=8 * 128, cols=96), N=128) == SHAPE
    assert call(W=desc(rows=8 * 120, cols=512, layout=1), N=120) == SHAPE  # tiled: N % 16


def test_moe_validation():
    L = q4.lib()
    B = A16
    # q4_moe_route(logits, ld, T, E, k, ids, weights, offsets, gather, inv, stream)
    assert L.q4_moe_route(B, 64, 256, 64, 0, B, B, B, B, B, None) == SHAPE
    assert L.q4_moe_route(B, 64, 256, 64, 65, B, B, B, B, B, None) == SHAPE
    assert L.q4_moe_route(B, 64, 256, 4, 8, B, B, B, B, B, None) == SHAPE      # k > E
    assert L.q4_moe_route(B, 2048, 256, 2048, 8, B, B, B, B, B, None) == SHAPE  # E > 1024
    assert L.q4_moe_route(B, 64, 20000, 64, 8, B, B, B, B, B, None) == SHAPE    # dispatch LDS
    assert L.q4_moe_route(B, 32, 256, 64, 8, B, B, B, B, B, None) == SHAPE      # ld < E
    assert L.q4_moe_route(None, 64, 256, 64, 8, B, B, B, B, B, None) == NULL
    assert L.q4_moe_route(B, 64, 256, 64, 8, B, B, None, B, B, None) == NULL
    assert L.q4_moe_route(B, 64, 256, 64, 8, B, B, B + 2, B, B, None) == ALIGN
    # q4_swiglu(gu, ld_gu, P, I, h, ldh, stream)
    assert L.q4_swiglu(B, 64, 8, 20, B, 32, None) == SHAPE                       # I % 8
    assert L.q4_swiglu(B, 60, 8, 32, B, 32, None) == SHAPE                       # ld_gu < 2I
    assert L.q4_swiglu(None, 64, 8, 32, B, 32, None) == NULL
    assert L.q4_swiglu(B, 64, 0, 32, B, 32, None) == OK
    # q4_moe_combine(y, ldy, inv, w, T, k, N, out, ldo, stream)
    assert L.q4_moe_combine(B, 64, B, B, 4, 2, 60, B, 64, None) == SHAPE          # N % 8
    assert L.q4_moe_combine(B, 64, B, B, 4, 0, 64, B, 64, None) == SHAPE
    assert L.q4_moe_combine(B, 64, None, B, 4, 2, 64, B, 64, None) == NULL
    assert L.q4_moe_combine(B, 64, B, B, 0, 2, 64, B, 64, None) == OK


def test_gemm_quantized_validation():
    L = q4.lib()
    T = q4.LAYOUT_TILED
    w = desc(rows=512, cols=512, layout=T)
    wmx = desc(rows=512, cols=512, layout=T)
    a = desc(rows=64, cols=512, layout=T)
    c = desc(rows=64, cols=512)                                   # MXFP4 output, row-major
    cn = desc(fmt=q4.NVFP4, rows=64, cols=512, gs=A16)            # NVFP4 output
    R = lambda *x: L.q4_gemm_quantized(*x, None)                  # noqa: E731
    by = ctypes.byref
    assert R(64, A16, 512, None, by(w), None, None) == NULL
    assert R(64, A16, 512, None, by(w), by(cn), None) == NULL                # NVFP4 needs a tensor scale
    assert R(64, A16, 512, None, by(w), by(c), A16) == FMT                   # only NVFP4 takes one
    assert R(64, A16, 512, None, by(w), by(cn), A_ODD) == ALIGN
    assert R(64, A16, 512, None, by(desc(rows=512, cols=512)), by(c), None) == FMT   # W must be tiled
    assert R(64, A16, 512, None, by(w), by(desc(fmt=q4.INT4_G128, rows=64, cols=512)), None) == FMT
    assert R(64, A16, 512, by(a), by(w), by(c), None) == FMT                 # both operands given
    assert R(64, None, 0, None, by(w), by(c), None) == NULL
    assert R(64, None, 0, by(desc(rows=64, cols=512)), by(wmx), by(c), None) == FMT    # A must be tiled
    assert R(64, None, 0, by(desc(fmt=q4.NVFP4, rows=64, cols=512, gs=A16, layout=T)),
             by(desc(fmt=q4.NVFP4, rows=512, cols=512, gs=A16, layout=T)), by(c), None) == FMT
    assert R(32, A16, 512, None, by(w), by(c), None) == SHAPE                # C rows != M
    assert R(64, A16, 512, None, by(w), by(desc(rows=64, cols=256)), None) == SHAPE
    assert R(64, A16, 512, None, by(desc(rows=48, cols=512, layout=T)),
             by(desc(fmt=q4.NVFP4, rows=64, cols=48, gs=A16)), A16) == SHAPE   # N % 32
    assert R(64, A16, 500, None, by(w), by(c), None) == SHAPE                # lda < K
    assert R(64, A_ODD, 512, None, by(w), by(c), None) == ALIGN
    assert R(32, None, 0, by(a), by(wmx), by(c), None) == SHAPE              # A rows != M
    assert R(0, A16, 512, None, by(w), by(desc(rows=0, cols=512)), None) == OK


def test_relayout_validation():
    """q4_relayout checks both descriptors and their agreement before any
    HIP call; an empty non-NVFP4 tensor is a no-op."""
    L = q4.lib()
    by = ctypes.byref
    T = 1
    src, dst = desc(cols=512), desc(cols=512, layout=T)
    assert L.q4_relayout(None, by(dst), None) == NULL
    assert L.q4_relayout(by(src), None, None) == NULL
    assert L.q4_relayout(by(src), by(desc(fmt=q4.INT4_G128, cols=512, layout=T)), None) == FMT
    assert L.q4_relayout(by(desc(fmt=q4.FP8_ROW, cols=512)), by(desc(fmt=q4.FP8_ROW, cols=512, layout=T)),
                         None) == FMT
    assert L.q4_relayout(by(src), by(desc(rows=48, cols=512, layout=T)), None) == SHAPE
    assert L.q4_relayout(by(desc(cols=256)), by(desc(cols=256, layout=T)), None) == SHAPE   # tiled: cols % 512
    assert L.q4_relayout(by(src), by(desc(cols=512, codes=A16 + 4, layout=T)), None) == ALIGN
    assert L.q4_relayout(by(desc(fmt=q4.NVFP4, cols=512)), by(desc(fmt=q4.NVFP4, cols=512, gs=A16, layout=T)),
                         None) == NULL                                      # src without its global scale
    assert L.q4_relayout(by(desc(rows=0, cols=512)), by(desc(rows=0, cols=512, layout=T)), None) == OK


def test_mfma_probe_validation():
    """Argument checks of the matrix-instruction probe; iters == 0 returns
    before any device query, so this runs without a GPU."""
    import ctypes
    L = q4.lib()
    f = ctypes.c_double(-1.0)
    assert L.q4_mfma_probe(7, 1, 0, A16, ctypes.byref(f), None) == FMT
    assert L.q4_mfma_probe(-1, 1, 0, A16, ctypes.byref(f), None) == FMT
    assert L.q4_mfma_probe(0, -1, 0, A16, ctypes.byref(f), None) == SHAPE
    assert L.q4_mfma_probe(0, (1 << 24) + 1, 0, A16, ctypes.byref(f), None) == SHAPE
    assert L.q4_mfma_probe(0, 1, 0, A16, None, None) == NULL
    assert L.q4_mfma_probe(1, 1, 0, None, ctypes.byref(f), None) == NULL
    assert L.q4_mfma_probe(1, 1, 0, A16 + 2, ctypes.byref(f), None) == ALIGN
    # the instruction-mix kinds copy 16 bytes per lane from the sink window
    assert L.q4_mfma_probe(4, 1, 0, A16 + 4, ctypes.byref(f), None) == ALIGN
    assert L.q4_mfma_probe(5, 1, 0, A16 + 8, ctypes.byref(f), None) == ALIGN
    assert L.q4_mfma_probe(6, 1, 0, A16 + 12, ctypes.byref(f), None) == ALIGN
    for kind in range(7):
        f.value = -1.0
        assert L.q4_mfma_probe(kind, 0, 0, None, ctypes.byref(f), None) == OK
        assert f.value == 0.0


def test_read_probe_validation():
    L = q4.lib()
    assert L.q4_read_probe(A16, 1000, A16, None) == SHAPE
    assert L.q4_read_probe(A16, -1024, A16, None) == SHAPE
    assert L.q4_read_probe(None, 1024, A16, None) == NULL
    assert L.q4_read_probe(A16, 1024, None, None) == NULL
    assert L.q4_read_probe(A16 + 4, 1024, A16, None) == ALIGN
    assert L.q4_read_probe(A16, 1024, A16 + 2, None) == ALIGN
    assert L.q4_read_probe(None, 0, None, None) == OK
