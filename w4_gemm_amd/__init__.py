"""w4_gemm_amd -- 4-bit absmax block quantization (INT4 g128, MXFP4, NVFP4)
and the W4 matmuls that consume it (W4A16, W4A4, W4A8 with per-token FP8
activations), as hand-written HIP kernels for gfx950.

This module is the thin Python binding of libq4.so's C ABI (include/q4.h):
the functions have the same names and only marshal arguments -- torch
tensors supply device memory and the current HIP stream, every step of the
computation runs in the library's kernels.  There is no CPU fallback: if the
library cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "INT4_G128", "MXFP4", "NVFP4", "FP8_ROW", "INT4_ZP", "FORMAT_NAMES", "GROUP", "Q4Error", "Q4Tensor",
    "LAYOUT_ROWS", "LAYOUT_TILED", "LAYOUT_NAMES",
    "lib", "q4_version", "q4_sizes", "q4_quantize", "q4_dequant", "q4_relayout", "relayout", "q4_gemv", "q4_gemm", "q4_gemm_quantized",
    "q4_grouped_gemm", "q4_grouped_gemm_swiglu", "q4_moe_route", "q4_swiglu", "q4_moe_combine",
    "moe_layer", "interleave_gate_up", "q4_read_probe", "q4_mfma_probe", "PROBE_KINDS", "PROBE_MIX_SINK",
    "empty_q4", "quantize", "LIB_PATH",
]

INT4_G128, MXFP4, NVFP4, FP8_ROW, INT4_ZP = 0, 1, 2, 3, 4
FORMAT_NAMES = {"int4": INT4_G128, "mxfp4": MXFP4, "nvfp4": NVFP4, "fp8_row": FP8_ROW, "int4_zp": INT4_ZP}
LAYOUT_ROWS, LAYOUT_TILED = 0, 1
LAYOUT_NAMES = {"rows": LAYOUT_ROWS, "tiled": LAYOUT_TILED}
GROUP = {INT4_G128: 128, MXFP4: 32, NVFP4: 16, FP8_ROW: 16, INT4_ZP: 128}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4.so")


class Q4Error(RuntimeError):
    def __init__(self, status: int, call: str):
        msg = _lib_handle().q4_status_string(status).decode() if _LIB else str(status)
        extra = ""
        if status == -6 and _LIB:
            extra = f" (hipError {_LIB.q4_last_hip_error()})"
        super().__init__(f"{call}: status {status}: {msg}{extra}")
        self.status = status


class _Q4TensorC(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("global_scale", ctypes.c_void_p),
    ]


_LIB = None


def _lib_handle():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            from . import _build
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32
        P = ctypes.POINTER(_Q4TensorC)
        sig = {
            "q4_version": ([], ctypes.c_int),
            "q4_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "q4_last_hip_error": ([], ctypes.c_int),
            "q4_sizes": ([ctypes.c_int, ctypes.c_int, i64, i64, ctypes.POINTER(ctypes.c_size_t),
                          ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
            "q4_quantize": ([vp, i64, P, vp, vp], ctypes.c_int),
            "q4_dequant": ([P, vp, ctypes.c_int, i64, vp], ctypes.c_int),
            "q4_relayout": ([P, P, vp], ctypes.c_int),
            "q4_gemv": ([P, vp, i64, i64, vp, i64, vp], ctypes.c_int),
            "q4_gemm": ([i64, vp, i64, P, P, vp, i64, vp], ctypes.c_int),
            "q4_gemm_quantized": ([i64, vp, i64, P, P, P, vp, vp], ctypes.c_int),
            "q4_grouped_gemm": ([vp, i64, i64, vp, vp, i32, i64, P, i64, vp, i64, vp],
                                ctypes.c_int),
            "q4_grouped_gemm_swiglu": ([vp, i64, i64, vp, vp, i32, i64, P, i64, vp, i64, vp],
                                       ctypes.c_int),
            "q4_moe_route": ([vp, i64, i64, i32, i32, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "q4_swiglu": ([vp, i64, i64, i64, vp, i64, vp], ctypes.c_int),
            "q4_moe_combine": ([vp, i64, vp, vp, i64, i32, i64, vp, i64, vp], ctypes.c_int),
            "q4_read_probe": ([vp, i64, vp, vp], ctypes.c_int),
            "q4_mfma_probe": ([ctypes.c_int32, i64, ctypes.c_uint32, vp, ctypes.POINTER(ctypes.c_double), vp],
                              ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _LIB = L
    return _LIB


def lib():
    """The loaded libq4.so (built in-tree first if it is missing)."""
    return _lib_handle()


def _check(status: int, call: str):
    if status != 0:
        raise Q4Error(status, call)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _on_gpu(*args):
    """Every tensor argument (or Q4Tensor buffer) is on the GPU.  Checked
    after the shapes, so that the shape checks can be tested on the CPU."""
    for name, t in args:
        if t is None:
            continue
        ts = ((f"{name}.codes", t.codes), (f"{name}.scales", t.scales),
              (f"{name}.global_scale", t.global_scale)) if isinstance(t, Q4Tensor) else ((name, t),)
        for n, x in ts:
            if x is not None and x.device.type != "cuda":
                raise ValueError(f"{n} must be a GPU tensor (got device {x.device})")


def _matrix(t: torch.Tensor, name: str, dtype, rows: int, cols: int, exact_cols: bool = False):
    """A 2-D argument with unit column stride, at least `rows` x `cols`
    (exactly `cols` columns if exact_cols).  Checked before any library
    call, so a wrong tensor never reaches a kernel as a pointer."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D (got shape {tuple(t.shape)})")
    if exact_cols and t.shape[1] != cols:
        raise ValueError(f"{name} must have {cols} columns (got {t.shape[1]})")
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{name} must be at least {rows} x {cols} (got {tuple(t.shape)})")
    if t.numel() and (t.stride(1) != 1 or (t.shape[0] > 1 and t.stride(0) < t.shape[1])):
        raise ValueError(f"{name} must have unit column stride and non-overlapping rows")


def _vector(t: torch.Tensor, name: str, dtype, n: int):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype:
        raise ValueError(f"{name} must be a {dtype} tensor")
    if not t.is_contiguous() or t.numel() < n:
        raise ValueError(f"{name} must be contiguous with at least {n} entries (got {t.numel()})")


def _q4(q: "Q4Tensor", name: str):
    """A quantized tensor's buffers: contiguous, as large as q4_sizes says
    for its format, layout and shape."""
    if not isinstance(q, Q4Tensor):
        raise ValueError(f"{name} must be a Q4Tensor")
    cb, sb = q4_sizes(q.fmt, q.rows, q.cols, q.layout)
    for part, t, need in (("codes", q.codes, cb), ("scales", q.scales, sb)):
        if not t.is_contiguous() or t.numel() * t.element_size() < need:
            raise ValueError(f"{name}.{part} must be contiguous and hold {need} bytes")
    if q.fmt == NVFP4:
        if q.global_scale is None:
            raise ValueError(f"{name}.global_scale is required for NVFP4")
        _vector(q.global_scale, f"{name}.global_scale", torch.float32, 1)


def _fmt(fmt) -> int:
    return FORMAT_NAMES[fmt] if isinstance(fmt, str) else int(fmt)


def _layout(layout) -> int:
    return LAYOUT_NAMES[layout] if isinstance(layout, str) else int(layout)


@dataclass
class Q4Tensor:
    """A quantized matrix: rows x cols values, blocks along cols.

    Row-major layout (LAYOUT_ROWS):
      codes  uint8 [rows, cols/2]   (even k in the low nibble)
      scales INT4: int16 (fp16 bits) [rows, cols/128]; MXFP4: uint8 (E8M0)
             [rows, cols/32]; NVFP4: uint8 (E4M3) [rows, cols/16]
    Tiled layout (LAYOUT_TILED, cols % 512 == 0): the same bytes arranged in
      16-row x 128-column tiles (include/q4.h); the tensors here are flat.
    global_scale  NVFP4: float32 [1] (dequant multiplier); else None
    FP8_ROW (W4A8 activations): codes uint8 [rows, cols] E4M3 (flat when
      tiled), scales float32 [rows].
    """
    fmt: int
    rows: int
    cols: int
    codes: torch.Tensor
    scales: torch.Tensor
    global_scale: Optional[torch.Tensor] = None
    layout: int = LAYOUT_ROWS

    def c(self) -> _Q4TensorC:
        return _Q4TensorC(self.fmt, self.layout, self.rows, self.cols,
                          self.codes.data_ptr() if self.codes.numel() else None,
                          self.scales.data_ptr() if self.scales.numel() else None,
                          None if self.global_scale is None else self.global_scale.data_ptr())

    @property
    def nbytes(self) -> int:
        n = self.codes.numel() + self.scales.numel() * self.scales.element_size()
        return n + (4 if self.global_scale is not None else 0)

    def clone(self) -> "Q4Tensor":
        return Q4Tensor(self.fmt, self.rows, self.cols, self.codes.clone(), self.scales.clone(),
                        None if self.global_scale is None else self.global_scale.clone(),
                        self.layout)


def q4_version() -> int:
    return lib().q4_version()


def q4_sizes(fmt, rows: int, cols: int, layout=LAYOUT_ROWS):
    """(codes bytes, scales bytes) of a rows x cols tensor."""
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().q4_sizes(_fmt(fmt), _layout(layout), rows, cols, ctypes.byref(cb),
                          ctypes.byref(sb)), "q4_sizes")
    return cb.value, sb.value


def empty_q4(fmt, rows: int, cols: int, device="cuda", layout=LAYOUT_ROWS) -> Q4Tensor:
    """Allocate (with torch) the buffers of a quantized tensor."""
    f, lay = _fmt(fmt), _layout(layout)
    cb, sb = q4_sizes(f, rows, cols, lay)
    if f == FP8_ROW:
        codes = torch.empty((rows, cols) if lay == LAYOUT_ROWS else (cb,), dtype=torch.uint8,
                            device=device)
        return Q4Tensor(f, rows, cols, codes, torch.empty(rows, dtype=torch.float32, device=device),
                        None, lay)
    g = GROUP[f]
    sdt = torch.int16 if f == INT4_G128 else torch.int32 if f == INT4_ZP else torch.uint8
    if lay == LAYOUT_ROWS:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((rows, cols // g), dtype=sdt, device=device)
    else:
        codes = torch.empty(cb, dtype=torch.uint8, device=device)
        scales = torch.empty(sb // torch.tensor([], dtype=sdt).element_size(), dtype=sdt, device=device)
    gs = torch.empty(1, dtype=torch.float32, device=device) if f == NVFP4 else None
    return Q4Tensor(f, rows, cols, codes, scales, gs, lay)


def q4_quantize(src: torch.Tensor, dst: Q4Tensor, nv_global_in: Optional[torch.Tensor] = None,
                stream=None) -> Q4Tensor:
    """Quantize bf16 src [rows, >= cols] (row stride src.stride(0)) into dst."""
    _matrix(src, "src", torch.bfloat16, dst.rows, dst.cols)
    _q4(dst, "dst")
    if nv_global_in is not None:
        _vector(nv_global_in, "nv_global_in", torch.float32, 1)
    _on_gpu(("src", src), ("dst", dst), ("nv_global_in", nv_global_in))
    desc = dst.c()
    _check(lib().q4_quantize(_ptr(src), src.stride(0), ctypes.byref(desc), _ptr(nv_global_in),
                             _stream(stream)), "q4_quantize")
    return dst


def quantize(src: torch.Tensor, fmt, nv_global_in: Optional[torch.Tensor] = None,
             stream=None, layout=LAYOUT_ROWS) -> Q4Tensor:
    """Allocate a Q4Tensor on src's device and quantize src into it."""
    dst = empty_q4(fmt, src.shape[0], src.shape[1], device=src.device, layout=layout)
    return q4_quantize(src, dst, nv_global_in, stream)


def q4_relayout(src: Q4Tensor, dst: Q4Tensor, stream=None) -> Q4Tensor:
    """Copy src into dst's layout (row-major <-> tiled), bit for bit; same
    format and shape.  The GEMM kernels want the tiled layout."""
    _q4(src, "src")
    _q4(dst, "dst")
    if src.fmt != dst.fmt or (src.rows, src.cols) != (dst.rows, dst.cols):
        raise ValueError("src and dst must have the same format and shape")
    _on_gpu(("src", src), ("dst", dst))
    a, b = src.c(), dst.c()
    _check(lib().q4_relayout(ctypes.byref(a), ctypes.byref(b), _stream(stream)), "q4_relayout")
    return dst


def relayout(src: Q4Tensor, layout=LAYOUT_TILED, stream=None) -> Q4Tensor:
    """Allocate a tensor of src's format and shape in `layout` and move src
    into it."""
    dst = empty_q4(src.fmt, src.rows, src.cols, device=src.codes.device, layout=layout)
    return q4_relayout(src, dst, stream)


def q4_dequant(src: Q4Tensor, dst: torch.Tensor, stream=None) -> torch.Tensor:
    """Dequantize into dst (bf16 or float32, [rows, >= cols])."""
    if dst.dtype == torch.bfloat16:
        dt = 0
    elif dst.dtype == torch.float32:
        dt = 1
    else:
        raise ValueError("dst must be bf16 or float32")
    _matrix(dst, "dst", dst.dtype, src.rows, src.cols)
    _q4(src, "src")
    _on_gpu(("src", src), ("dst", dst))
    desc = src.c()
    _check(lib().q4_dequant(ctypes.byref(desc), _ptr(dst), dt, dst.stride(0), _stream(stream)),
           "q4_dequant")
    return dst


def q4_gemv(W: Q4Tensor, x: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """y[b, n] = sum_k x[b, k] w'[n, k] for b < x.shape[0] (<= 16)."""
    _q4(W, "W")
    _matrix(x, "x", torch.bfloat16, 0, W.cols, exact_cols=True)
    _matrix(y, "y", torch.bfloat16, x.shape[0], W.rows)
    _on_gpu(("W", W), ("x", x), ("y", y))
    desc = W.c()
    _check(lib().q4_gemv(ctypes.byref(desc), _ptr(x), x.shape[0], x.stride(0), _ptr(y),
                         y.stride(0), _stream(stream)), "q4_gemv")
    return y


def q4_gemm(A, W: Q4Tensor, C: torch.Tensor, stream=None) -> torch.Tensor:
    """C = A' W'^T.  A is a bf16 tensor [M, K] (W4A16), an MXFP4 or NVFP4
    Q4Tensor (W4A4, with W in the same format) or an FP8_ROW Q4Tensor (W4A8,
    with W INT4)."""
    _q4(W, "W")
    if isinstance(A, Q4Tensor):
        _q4(A, "A")
        if A.cols != W.cols:
            raise ValueError(f"A has {A.cols} columns, W {W.cols}")
        M = A.rows
    else:
        _matrix(A, "A", torch.bfloat16, 0, W.cols, exact_cols=True)
        M = A.shape[0]
    _matrix(C, "C", torch.bfloat16, M, W.rows)
    _on_gpu(("W", W), ("A", A), ("C", C))
    wd = W.c()
    if isinstance(A, Q4Tensor):
        ad = A.c()
        st = lib().q4_gemm(A.rows, None, 0, ctypes.byref(ad), ctypes.byref(wd), _ptr(C),
                           C.stride(0), _stream(stream))
    else:
        st = lib().q4_gemm(A.shape[0], _ptr(A), A.stride(0), None, ctypes.byref(wd), _ptr(C),
                           C.stride(0), _stream(stream))
    _check(st, "q4_gemm")
    return C


def q4_gemm_quantized(A, W: Q4Tensor, C: Q4Tensor, nv_global_in: Optional[torch.Tensor] = None,
                      stream=None) -> Q4Tensor:
    """The GEMM of q4_gemm with C written quantized by its epilogue (MXFP4,
    or NVFP4 with the tensor scale nv_global_in): C holds what q4_quantize
    writes for the bf16 product.  A is bf16 [M, K] (W tiled, any weight
    format) or an MXFP4 tiled Q4Tensor (W MXFP4 tiled)."""
    _q4(W, "W")
    _q4(C, "C")
    if isinstance(A, Q4Tensor):
        _q4(A, "A")
        if A.cols != W.cols:
            raise ValueError(f"A has {A.cols} columns, W {W.cols}")
        M = A.rows
    else:
        _matrix(A, "A", torch.bfloat16, 0, W.cols, exact_cols=True)
        M = A.shape[0]
    if C.rows != M or C.cols != W.rows:
        raise ValueError(f"C must be {M} x {W.rows} (got {C.rows} x {C.cols})")
    if nv_global_in is not None:
        _vector(nv_global_in, "nv_global_in", torch.float32, 1)
    _on_gpu(("W", W), ("A", A), ("C", C), ("nv_global_in", nv_global_in))
    wd, cd = W.c(), C.c()
    if isinstance(A, Q4Tensor):
        ad = A.c()
        st = lib().q4_gemm_quantized(M, None, 0, ctypes.byref(ad), ctypes.byref(wd), ctypes.byref(cd),
                                     _ptr(nv_global_in), _stream(stream))
    else:
        st = lib().q4_gemm_quantized(M, _ptr(A), A.stride(0), None, ctypes.byref(wd), ctypes.byref(cd),
                                     _ptr(nv_global_in), _stream(stream))
    _check(st, "q4_gemm_quantized")
    return C


def q4_grouped_gemm(A: torch.Tensor, gather: torch.Tensor, offsets: torch.Tensor, W: Q4Tensor,
                    N: int, C: torch.Tensor, stream=None) -> torch.Tensor:
    """For expert e, rows p in [offsets[e], offsets[e+1]):
    C[p] = A[gather[p]] . w'_e^T, with W stacked expert-major (E*N rows).
    gather None: row p reads A[p] (P = C.shape[0] rows)."""
    _q4(W, "W")
    _matrix(A, "A", torch.bfloat16, 0, W.cols, exact_cols=True)
    _vector(offsets, "offsets", torch.int32, 1)
    E = offsets.numel() - 1
    if W.rows != E * N:
        raise ValueError(f"W has {W.rows} rows, not experts ({E}) x N ({N})")
    if gather is not None:
        _vector(gather, "gather", torch.int32, 0)
    P = C.shape[0] if gather is None else gather.numel()
    _matrix(C, "C", torch.bfloat16, P, N)
    _on_gpu(("W", W), ("A", A), ("gather", gather), ("offsets", offsets), ("C", C))
    wd = W.c()
    _check(lib().q4_grouped_gemm(_ptr(A), A.stride(0), A.shape[0], _ptr(gather), _ptr(offsets),
                                 E, P, ctypes.byref(wd), N, _ptr(C), C.stride(0),
                                 _stream(stream)), "q4_grouped_gemm")
    return C


@dataclass
class Routing:
    """Device tensors written by q4_moe_route (see include/q4.h)."""
    ids: torch.Tensor        # int32 [T, k]
    weights: torch.Tensor    # float32 [T, k]
    offsets: torch.Tensor    # int32 [E + 1]
    gather: torch.Tensor     # int32 [T * k]
    inv: torch.Tensor        # int32 [T, k]


def q4_moe_route(logits: torch.Tensor, k: int, stream=None) -> Routing:
    """Top-k routing with softmax gates and the expert-major dispatch order
    for fp32 router logits [T, E] (unit column stride)."""
    _matrix(logits, "logits", torch.float32, 0, 0)
    _on_gpu(("logits", logits))
    T, E = logits.shape
    dev = logits.device
    r = Routing(torch.empty((T, k), dtype=torch.int32, device=dev),
                torch.empty((T, k), dtype=torch.float32, device=dev),
                torch.empty(E + 1, dtype=torch.int32, device=dev),
                torch.empty(T * k, dtype=torch.int32, device=dev),
                torch.empty((T, k), dtype=torch.int32, device=dev))
    _check(lib().q4_moe_route(_ptr(logits), logits.stride(0) if T else E, T, E, k, _ptr(r.ids), _ptr(r.weights),
                              _ptr(r.offsets), _ptr(r.gather), _ptr(r.inv), _stream(stream)),
           "q4_moe_route")
    return r


def q4_swiglu(gu: torch.Tensor, inter: int, h: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """h = silu(gu[:, :inter]) * gu[:, inter:2*inter] (bf16)."""
    _matrix(gu, "gu", torch.bfloat16, 0, 2 * inter)
    P = gu.shape[0]
    if h is None:
        h = torch.empty((P, inter), dtype=torch.bfloat16, device=gu.device)
    _matrix(h, "h", torch.bfloat16, P, inter)
    _on_gpu(("gu", gu), ("h", h))
    _check(lib().q4_swiglu(_ptr(gu), gu.stride(0), P, inter, _ptr(h), h.stride(0), _stream(stream)),
           "q4_swiglu")
    return h


def q4_moe_combine(y: torch.Tensor, r: Routing, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """out[t] = sum_j r.weights[t, j] * y[r.inv[t, j]] (bf16)."""
    T, k = r.inv.shape
    _vector(r.inv, "r.inv", torch.int32, T * k)
    _vector(r.weights, "r.weights", torch.float32, T * k)
    _matrix(y, "y", torch.bfloat16, T * k, 0)
    N = y.shape[1]
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=y.device)
    _matrix(out, "out", torch.bfloat16, T, N)
    _on_gpu(("y", y), ("r.inv", r.inv), ("r.weights", r.weights), ("out", out))
    _check(lib().q4_moe_combine(_ptr(y), y.stride(0), _ptr(r.inv), _ptr(r.weights), T, k, N, _ptr(out),
                                out.stride(0), _stream(stream)), "q4_moe_combine")
    return out


def q4_grouped_gemm_swiglu(A: torch.Tensor, gather: Optional[torch.Tensor], offsets: torch.Tensor,
                           W: Q4Tensor, inter: int, H: torch.Tensor, stream=None) -> torch.Tensor:
    """H[p] = silu(A[gather[p]] . W_gate_e^T) * (A[gather[p]] . W_up_e^T),
    with W's 2*inter rows per expert alternating 16-row gate and up tiles
    (see interleave_gate_up); gather None: row p reads A[p]."""
    _q4(W, "W")
    _matrix(A, "A", torch.bfloat16, 0, W.cols, exact_cols=True)
    _vector(offsets, "offsets", torch.int32, 1)
    E = offsets.numel() - 1
    if W.rows != E * 2 * inter:
        raise ValueError(f"W has {W.rows} rows, not experts ({E}) x 2 x inter ({inter})")
    if gather is not None:
        _vector(gather, "gather", torch.int32, 0)
    P = H.shape[0] if gather is None else gather.numel()
    _matrix(H, "H", torch.bfloat16, P, inter)
    _on_gpu(("W", W), ("A", A), ("gather", gather), ("offsets", offsets), ("H", H))
    wd = W.c()
    _check(lib().q4_grouped_gemm_swiglu(_ptr(A), A.stride(0), A.shape[0], _ptr(gather), _ptr(offsets), E, P,
                                        ctypes.byref(wd), inter, _ptr(H), H.stride(0), _stream(stream)),
           "q4_grouped_gemm_swiglu")
    return H


def q4_read_probe(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Measurement helper: stream-read all of src (a contiguous GPU tensor of
    a multiple of 1024 bytes) and discard it (sink: int32 GPU tensor [1])."""
    if not isinstance(src, torch.Tensor) or not src.is_contiguous():
        raise ValueError("src must be a contiguous tensor")
    nbytes = src.numel() * src.element_size()
    if nbytes % 1024:
        raise ValueError("src must hold a multiple of 1024 bytes")
    _vector(sink, "sink", torch.int32, 1)
    _on_gpu(("src", src), ("sink", sink))
    _check(lib().q4_read_probe(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "q4_read_probe")


PROBE_KINDS = {"fp4": 0, "bf16": 1, "fp16": 2, "fp8": 3, "fp4_copy": 4, "fp4_mix": 5, "bf16_mix": 6}
PROBE_MIX_SINK = 16384   # int32 entries the "fp4_copy" / "fp4_mix" / "bf16_mix" kinds read (64 KB)


def q4_mfma_probe(kind: str, iters: int, sink: torch.Tensor, seed: int = 1, stream=None) -> float:
    """Measurement helper: back-to-back matrix instructions of one kind
    ("fp4", "bf16", "fp16", "fp8") on random register operands, or the FP4
    instruction with the tiled W4A4 kernel's global->LDS copies
    ("fp4_copy") or its copies and LDS fragment reads ("fp4_mix") mixed in,
    or the bf16 instruction with the tiled W4A16 GEMM's NVFP4 dequantization,
    copies and fragment reads ("bf16_mix"); returns the launch's
    floating-point operations.  sink: int32 GPU tensor [1] ([PROBE_MIX_SINK],
    16-byte aligned, for the three mix kinds)."""
    if kind not in PROBE_KINDS:
        raise ValueError(f"kind must be one of {sorted(PROBE_KINDS)}")
    if not isinstance(iters, int) or iters < 0 or iters > (1 << 24):
        raise ValueError("iters must be an int in [0, 2^24]")
    _vector(sink, "sink", torch.int32, PROBE_MIX_SINK if PROBE_KINDS[kind] >= 4 else 1)
    _on_gpu(("sink", sink))
    flops = ctypes.c_double(0.0)
    _check(lib().q4_mfma_probe(PROBE_KINDS[kind], iters, seed & 0xFFFFFFFF, _ptr(sink), ctypes.byref(flops),
                               _stream(stream)), "q4_mfma_probe")
    return flops.value


def interleave_gate_up(w_gu: torch.Tensor, experts: int, inter: int) -> torch.Tensor:
    """[W_gate_e; W_up_e] per expert (2*inter rows each) -> the row order
    q4_grouped_gemm_swiglu takes: 16-row tiles alternating gate and up
    (a permutation of rows, done before quantization)."""
    K = w_gu.shape[1]
    w = w_gu.reshape(experts, 2, inter // 16, 16, K)       # expert, gate/up, tile, row, k
    return w.permute(0, 2, 1, 3, 4).reshape(experts * 2 * inter, K).contiguous()


def moe_layer(x: torch.Tensor, logits: torch.Tensor, k: int, W_gu: Q4Tensor, W_down: Q4Tensor,
              inter: int, stream=None, fused: bool = False):
    """One MoE FFN layer: route, gate/up grouped GEMM, SwiGLU, down grouped
    GEMM, combine -- library calls on the same stream.  W_gu holds
    [W_gate_e; W_up_e] (2*inter rows) per expert, or with fused=True the
    interleave_gate_up order (then q4_grouped_gemm_swiglu makes h directly);
    W_down has K rows per expert.  Returns (out [T, K] bf16, Routing)."""
    T, K = x.shape
    r = q4_moe_route(logits, k, stream)
    P = T * k
    if fused:
        h = torch.empty((P, inter), dtype=torch.bfloat16, device=x.device)
        q4_grouped_gemm_swiglu(x, r.gather, r.offsets, W_gu, inter, h, stream)
    else:
        gu = torch.empty((P, 2 * inter), dtype=torch.bfloat16, device=x.device)
        q4_grouped_gemm(x, r.gather, r.offsets, W_gu, 2 * inter, gu, stream)
        h = q4_swiglu(gu, inter, stream=stream)
    y = torch.empty((P, K), dtype=torch.bfloat16, device=x.device)
    q4_grouped_gemm(h, None, r.offsets, W_down, K, y, stream)
    return q4_moe_combine(y, r, stream=stream), r
