"""CPU oracle for 4-bit absmax block quantization and the W4 matmuls.

TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP
library (w4_gemm_amd) and neither imports the other.

The quantizers and dequantizers are plain C (q4_oracle.c, fp32 steps exactly
as each format is stated on the pages; see the header of that file for the
passages and the readings).  The matmul references below are the plain
definitions in fp64 on the oracle's own dequantized weights:

  * W4A16 GEMV / GEMM: out[m, n] = sum_k a[m, k] * w'[n, k]  -- the matmul
    the W4A16 scheme performs after dequantizing weights ("Low-bit inference
    for very large MoE", table "Kernels on different hardware", row W4A16).
  * W4A4 MXFP4: both operands MXFP4-quantized along K, then the same sum on
    the dequantized values (same table, row W4A4).
  * W4A8: INT4 weights, activations quantized to FP8 E4M3 with one scale
    per token (formats.py fp8_per_row, "Quantization in deployment"), then
    the same sum on both dequantized operands (same table, row W4A8).
  * Grouped MoE GEMM: one low-bit weight matrix per expert, each routed row
    multiplied by its expert's matrix (same page, "A few details", MoE
    grouped GEMM bullet).
  * The MoE layer around it: top-k routing with softmax gates, SwiGLU
    expert FFN (gate/up grouped GEMM, silu(gate) * up, down grouped GEMM)
    and the gated combine -- plain definitions in fp64 (readings stated in
    the functions).

numpy's fp64 matmul is the only library primitive used as a step.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

FORMATS = ("int4", "mxfp4", "nvfp4", "int4_zp")
GROUP = {"int4": 128, "mxfp4": 32, "nvfp4": 16, "int4_zp": 128}

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def lib():
    """Load liboracle.so, building it with gcc first if it is not there."""
    global _LIB
    if _LIB is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_e2m1_code.argtypes = [ctypes.c_float]
        L.oracle_e2m1_code.restype = ctypes.c_int
        L.oracle_e2m1_value.argtypes = [ctypes.c_int]
        L.oracle_e2m1_value.restype = ctypes.c_float
        L.oracle_e4m3_code.argtypes = [ctypes.c_float]
        L.oracle_e4m3_code.restype = ctypes.c_int
        L.oracle_e4m3_value.argtypes = [ctypes.c_int]
        L.oracle_e4m3_value.restype = ctypes.c_float
        L.oracle_fp16_code.argtypes = [ctypes.c_float]
        L.oracle_fp16_code.restype = ctypes.c_int
        L.oracle_fp16_value.argtypes = [ctypes.c_int]
        L.oracle_fp16_value.restype = ctypes.c_float
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_set_ties_toward_zero.argtypes = [ctypes.c_int]
        L.oracle_set_ties_toward_zero.restype = None
        L.oracle_absmax_int_group.argtypes = [_p, _i64, ctypes.c_int, _p]
        L.oracle_absmax_int_group.restype = ctypes.c_int
        L.oracle_mx_scale_exponent.argtypes = [ctypes.c_float]
        L.oracle_mx_scale_exponent.restype = ctypes.c_int
        L.oracle_nv_block_scale_code.argtypes = [ctypes.c_float, ctypes.c_float]
        L.oracle_nv_block_scale_code.restype = ctypes.c_int
        L.oracle_nv_global_scale.argtypes = [_p, _i64, _i64, _i64]
        L.oracle_nv_global_scale.restype = ctypes.c_float
        L.oracle_quantize_int4.argtypes = [_p, _i64, _i64, _i64, _i64, _p, _p]
        L.oracle_quantize_int4.restype = ctypes.c_int
        L.oracle_quantize_mxfp4.argtypes = [_p, _i64, _i64, _i64, _p, _p]
        L.oracle_quantize_mxfp4.restype = ctypes.c_int
        L.oracle_quantize_nvfp4.argtypes = [_p, _i64, _i64, _i64, _p, _p, _p, _p]
        L.oracle_quantize_nvfp4.restype = ctypes.c_int
        L.oracle_fp8_row_scale.argtypes = [ctypes.c_float]
        L.oracle_fp8_row_scale.restype = ctypes.c_float
        L.oracle_fp8_code.argtypes = [ctypes.c_float, ctypes.c_float]
        L.oracle_fp8_code.restype = ctypes.c_int
        L.oracle_quantize_fp8_rows.argtypes = [_p, _i64, _i64, _i64, _p, _p]
        L.oracle_quantize_fp8_rows.restype = None
        L.oracle_dequant_fp8_rows.argtypes = [_p, _p, _i64, _i64, _p]
        L.oracle_dequant_fp8_rows.restype = None
        L.oracle_int4zp_group.argtypes = [_p, _i64, _p]
        L.oracle_int4zp_group.restype = ctypes.c_uint32
        L.oracle_quantize_int4zp.argtypes = [_p, _i64, _i64, _i64, _p, _p]
        L.oracle_quantize_int4zp.restype = ctypes.c_int
        L.oracle_dequant_int4zp.argtypes = [_p, _p, _i64, _i64, _p]
        L.oracle_dequant_int4zp.restype = None
        L.oracle_dequant_int4.argtypes = [_p, _p, _i64, _i64, _i64, _p]
        L.oracle_dequant_int4.restype = None
        L.oracle_dequant_mxfp4.argtypes = [_p, _p, _i64, _i64, _p]
        L.oracle_dequant_mxfp4.restype = None
        L.oracle_dequant_nvfp4.argtypes = [_p, _p, ctypes.c_float, _i64, _i64, _p]
        L.oracle_dequant_nvfp4.restype = None
        L.oracle_f32_to_bf16_array.argtypes = [_p, _i64, _p]
        L.oracle_f32_to_bf16_array.restype = None
        _LIB = L
    return _LIB


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(w) -> np.ndarray:
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float32))
    if w.ndim != 2:
        raise ValueError("expected a 2-D array")
    return w


# --------------------------------------------------------------------------
# single-value helpers (pins)
# --------------------------------------------------------------------------
def e2m1_code(a: float) -> int:
    return lib().oracle_e2m1_code(a)


def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(code)


def e4m3_code(t: float) -> int:
    return lib().oracle_e4m3_code(t)


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(code)


def fp16_code(t: float) -> int:
    return lib().oracle_fp16_code(t)


def fp16_value(code: int) -> float:
    return lib().oracle_fp16_value(code)


def mx_scale_exponent(amax: float) -> int:
    return lib().oracle_mx_scale_exponent(amax)


def nv_block_scale_code(amax_b: float, gs: float) -> int:
    return lib().oracle_nv_block_scale_code(amax_b, gs)


def set_ties_toward_zero(on: bool) -> None:
    """Test-only switch: exact E2M1 ties go to the lower neighbour (what the
    argmin of formats.py fp4() returns, "Quantization in deployment", Fake
    quantization) instead of the even code.  E4M3, fp16 and INT4 roundings
    keep ties to even either way, as formats.py's float8_e4m3fn cast and
    fake_int4's torch.round do."""
    lib().oracle_set_ties_toward_zero(1 if on else 0)


def absmax_int_group(w, qmax: int):
    """One symmetric absmax group: (fp16 scale code, integer codes)."""
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float32).ravel())
    q = np.zeros(w.size, dtype=np.int32)
    code = lib().oracle_absmax_int_group(_ptr(w), w.size, qmax, _ptr(q))
    return code, q


def f32_to_bf16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f32_to_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# quantize / dequantize
# --------------------------------------------------------------------------
class QTensor:
    """Oracle-side quantized tensor: packed codes, raw scale bytes, gs."""

    def __init__(self, fmt, rows, cols, codes, scales, gs=None):
        self.fmt, self.rows, self.cols = fmt, rows, cols
        self.codes, self.scales, self.gs = codes, scales, gs


def quantize(fmt: str, w, gs: float | None = None) -> QTensor:
    w = _f32(w)
    rows, cols = w.shape
    g = GROUP[fmt]
    if cols % g:
        raise ValueError(f"cols {cols} is not a multiple of {g}")
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    L = lib()
    if fmt == "int4":
        scales = np.zeros((rows, cols // g), dtype=np.uint16)
        rc = L.oracle_quantize_int4(_ptr(w), rows, cols, cols, g, _ptr(codes), _ptr(scales))
        out_gs = None
    elif fmt == "mxfp4":
        scales = np.zeros((rows, cols // g), dtype=np.uint8)
        rc = L.oracle_quantize_mxfp4(_ptr(w), rows, cols, cols, _ptr(codes), _ptr(scales))
        out_gs = None
    elif fmt == "int4_zp":
        scales = np.zeros((rows, cols // g), dtype=np.uint32)
        rc = L.oracle_quantize_int4zp(_ptr(w), rows, cols, cols, _ptr(codes), _ptr(scales))
        out_gs = None
    elif fmt == "nvfp4":
        scales = np.zeros((rows, cols // g), dtype=np.uint8)
        gs_out = np.zeros(1, dtype=np.float32)
        gs_in = None if gs is None else np.array([gs], dtype=np.float32)
        rc = L.oracle_quantize_nvfp4(_ptr(w), rows, cols, cols,
                                     None if gs_in is None else _ptr(gs_in),
                                     _ptr(codes), _ptr(scales), _ptr(gs_out))
        out_gs = float(gs_out[0])
    else:
        raise ValueError(fmt)
    if rc != 0:
        raise ValueError(f"oracle quantize failed ({rc})")
    return QTensor(fmt, rows, cols, codes, scales, out_gs)


def int4zp_group(w):
    """(scale word, codes) of one group of INT4 with a zero point."""
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float32))
    q = np.zeros(len(w), dtype=np.int32)
    word = int(lib().oracle_int4zp_group(_ptr(w), len(w), _ptr(q)))
    return word, q


def nv_global_scale(w) -> float:
    w = _f32(w)
    return float(lib().oracle_nv_global_scale(_ptr(w), w.shape[0], w.shape[1], w.shape[1]))


def dequant(q: QTensor) -> np.ndarray:
    """fp32 dequantized values: fp32(code value * scale as stored)."""
    out = np.empty((q.rows, q.cols), dtype=np.float32)
    codes = np.ascontiguousarray(q.codes)
    scales = np.ascontiguousarray(q.scales)
    L = lib()
    if q.fmt == "int4":
        L.oracle_dequant_int4(_ptr(codes), _ptr(scales), q.rows, q.cols, 128, _ptr(out))
    elif q.fmt == "mxfp4":
        L.oracle_dequant_mxfp4(_ptr(codes), _ptr(scales), q.rows, q.cols, _ptr(out))
    elif q.fmt == "int4_zp":
        L.oracle_dequant_int4zp(_ptr(codes), _ptr(scales), q.rows, q.cols, _ptr(out))
    else:
        L.oracle_dequant_nvfp4(_ptr(codes), _ptr(scales), q.gs, q.rows, q.cols, _ptr(out))
    return out


def dequant_rows(q: QTensor, rows) -> np.ndarray:
    """Dequantize a subset of rows (for sampled checks at full size)."""
    rows = np.asarray(rows, dtype=np.int64)
    sub = QTensor(q.fmt, len(rows), q.cols, np.ascontiguousarray(q.codes[rows]),
                  np.ascontiguousarray(q.scales[rows]), q.gs)
    return dequant(sub)


# --------------------------------------------------------------------------
# matmul references (fp64)
# --------------------------------------------------------------------------
def matmul_f64(a, w_deq) -> np.ndarray:
    """out[m, n] = sum_k a[m, k] * w'[n, k], in fp64."""
    a64 = np.asarray(a, dtype=np.float64)
    w64 = np.asarray(w_deq, dtype=np.float64)
    return a64 @ w64.T


def gemv(q: QTensor, x) -> np.ndarray:
    """W4A16 GEMV: y[b, n] = sum_k x[b, k] * w'[n, k] (fp64)."""
    return matmul_f64(x, dequant(q))


def gemm_w4a16(a, q: QTensor, rows=None) -> np.ndarray:
    """W4A16 GEMM C = A w'^T (fp64); `rows` selects output rows of C."""
    a = np.asarray(a, dtype=np.float32)
    if rows is not None:
        a = a[np.asarray(rows)]
    return matmul_f64(a, dequant(q))


def gemm_w4a4(a, q: QTensor, rows=None, aq: QTensor | None = None) -> np.ndarray:
    """W4A4 GEMM: C = deq(fmt(A)) deq(W)^T (fp64), both operands in the
    weight's FP4 format ("Low-bit inference for very large MoE", table
    "Kernels on different hardware", row W4A4; "Quantization in deployment",
    the MXFP4 and NVFP4 rows of the cheat sheet).  MXFP4: E8M0 per 32.
    NVFP4: E4M3 per 16 and A's own tensor global scale, computed from the
    whole of A (so a row subset must come with the full-A quantization `aq`,
    or the full A)."""
    if q.fmt not in ("mxfp4", "nvfp4"):
        raise ValueError("W4A4 is defined for MXFP4 and NVFP4 operands")
    if aq is None:
        a = _f32(a)
        if rows is not None and q.fmt == "mxfp4":   # row-local scales: quantize the rows only
            aq = quantize("mxfp4", np.ascontiguousarray(a[np.asarray(rows)]))
            rows = None
        else:
            aq = quantize(q.fmt, a)
    if aq.fmt != q.fmt:
        raise ValueError("W4A4 takes both operands in one format")
    if rows is not None:
        aq = QTensor(aq.fmt, len(rows), aq.cols, aq.codes[np.asarray(rows)],
                     aq.scales[np.asarray(rows)], aq.gs)
    return matmul_f64(dequant(aq), dequant(q))


class FP8Rows:
    """Oracle-side FP8 activations: E4M3 codes [rows, cols] (row-major) and
    one fp32 scale per row."""

    def __init__(self, rows, cols, codes, scales):
        self.rows, self.cols, self.codes, self.scales = rows, cols, codes, scales


def quantize_fp8_rows(a) -> FP8Rows:
    """Per-token FP8 quantization (formats.py fp8_per_row, "Quantization in
    deployment"): scale = max(amax_row, 1e-12)/448, E4M3 of clamp(x/scale)."""
    a = _f32(a)
    rows, cols = a.shape
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scales = np.zeros(rows, dtype=np.float32)
    lib().oracle_quantize_fp8_rows(_ptr(a), rows, cols, cols, _ptr(codes), _ptr(scales))
    return FP8Rows(rows, cols, codes, scales)


def fp8_row_scale(amax: float) -> float:
    return float(lib().oracle_fp8_row_scale(float(amax)))


def fp8_code(x: float, s: float) -> int:
    return int(lib().oracle_fp8_code(float(x), float(s)))


def dequant_fp8_rows(q: FP8Rows) -> np.ndarray:
    """fp32(E4M3 value * row scale)."""
    out = np.empty((q.rows, q.cols), dtype=np.float32)
    codes = np.ascontiguousarray(q.codes)
    scales = np.ascontiguousarray(q.scales, dtype=np.float32)
    lib().oracle_dequant_fp8_rows(_ptr(codes), _ptr(scales), q.rows, q.cols, _ptr(out))
    return out


def gemm_w4a8(a, q: QTensor, rows=None, aq: FP8Rows | None = None) -> np.ndarray:
    """W4A8 GEMM: C = deq(fp8_per_row(A)) deq(W)^T in fp64, W INT4 g128
    ("Low-bit inference for very large MoE", table "Kernels on different
    hardware", row W4A8: INT4 weights, activations quantized to FP8)."""
    if q.fmt != "int4":
        raise ValueError("W4A8 is defined for INT4 weights")
    if aq is None:
        a = _f32(a)
        if rows is not None:
            a = np.ascontiguousarray(a[np.asarray(rows)])
        aq = quantize_fp8_rows(a)
    elif rows is not None:
        r = np.asarray(rows)
        aq = FP8Rows(len(r), aq.cols, aq.codes[r], aq.scales[r])
    return matmul_f64(dequant_fp8_rows(aq), dequant(q))


# --------------------------------------------------------------------------
# MoE layer around the grouped GEMM (routing, SwiGLU, combine)
# --------------------------------------------------------------------------
class Routing:
    """Top-k routing of T tokens over E experts: ids/weights [T, k] (choice j
    = j-th largest logit, ties to the lower expert id), expert offsets [E+1],
    gather [T*k] (token of each routed row; rows expert-major, tokens
    ascending within an expert) and inv [T, k] (routed row of each choice)."""

    def __init__(self, ids, weights, offsets, gather, inv):
        self.ids, self.weights, self.offsets, self.gather, self.inv = ids, weights, offsets, gather, inv


def moe_route(logits, k: int) -> Routing:
    """Routing for one MoE layer: each token goes to the k experts with the
    largest router logits (ties to the lower expert id); its gate for a
    chosen expert is that expert's softmax probability over all E logits
    (fp64), not renormalized over the k.  Rows are then grouped by expert
    ("Low-bit inference for very large MoE", "A few details": one low-bit
    matrix per expert, tokens grouped by routing)."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.zeros((T, k), dtype=np.int32)
    weights = np.zeros((T, k), dtype=np.float64)
    l64 = lg.astype(np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))
        ids[t] = order[:k]
        z = np.exp(l64[t] - l64[t].max())
        p = z / z.sum()
        weights[t] = p[ids[t]]
    counts = np.bincount(ids.ravel(), minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    gather = np.zeros(T * k, dtype=np.int32)
    inv = np.zeros((T, k), dtype=np.int32)
    nxt = offsets[:-1].copy()
    for t in range(T):          # tokens ascending: stable within each expert
        for e in sorted(ids[t]):
            j = int(np.where(ids[t] == e)[0][0])
            gather[nxt[e]] = t
            inv[t, j] = nxt[e]
            nxt[e] += 1
    return Routing(ids, weights, offsets, gather, inv)


def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), fp64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(gu, inter: int) -> np.ndarray:
    """SwiGLU of a gate/up product row: h = silu(gate) * up, where gate is
    columns [0, inter) and up columns [inter, 2*inter) of gu (fp64)."""
    gu = np.asarray(gu, dtype=np.float64)
    return silu(gu[:, :inter]) * gu[:, inter:2 * inter]


def moe_combine(y, inv, weights) -> np.ndarray:
    """out[t] = sum_j weights[t, j] * y[inv[t, j]] (fp64)."""
    y = np.asarray(y, dtype=np.float64)
    inv = np.asarray(inv)
    w = np.asarray(weights, dtype=np.float64)
    return np.einsum("tj,tjn->tn", w, y[inv])


def moe_layer(x, logits, k: int, q_gu: QTensor, q_down: QTensor, inter: int, tokens=None):
    """One MoE FFN layer in fp64 on the oracle's dequantized weights:
    out[t] = sum_j g_tj * W_down_e (silu(W_gate_e x_t) * (W_up_e x_t)),
    e = the token's j-th expert, with W_gu_e = [W_gate_e; W_up_e] rows
    [e*2I, (e+1)*2I) of q_gu and W_down_e rows [e*K, (e+1)*K) of q_down.
    Returns (out [len(tokens), K], Routing)."""
    x = np.asarray(x, dtype=np.float32)
    r = moe_route(logits, k)
    K = x.shape[1]
    tokens = range(x.shape[0]) if tokens is None else tokens
    out = np.zeros((len(tokens), K), dtype=np.float64)
    cache = {}
    for i, t in enumerate(tokens):
        for j in range(k):
            e = int(r.ids[t, j])
            if e not in cache:
                cache[e] = (dequant_rows(q_gu, np.arange(e * 2 * inter, (e + 1) * 2 * inter)).astype(np.float64),
                            dequant_rows(q_down, np.arange(e * K, (e + 1) * K)).astype(np.float64))
            wgu, wd = cache[e]
            gu = wgu @ x[t].astype(np.float64)
            h = silu(gu[:inter]) * gu[inter:]
            out[i] += r.weights[t, j] * (wd @ h)
    return out, r


def grouped_gemm(a, gather, offsets, q_all: QTensor, n: int, experts=None) -> np.ndarray:
    """Grouped expert GEMM: for expert e, rows p in [offsets[e], offsets[e+1])
    get C[p] = a[gather[p]] . w'_e^T, where w'_e is rows [e*n, (e+1)*n) of
    the expert-major quantized weight.  Returns fp64 [P, n]; rows of experts
    not listed in `experts` (when given) are left NaN."""
    a = np.asarray(a, dtype=np.float32)
    gather = np.asarray(gather)
    offsets = np.asarray(offsets)
    E = len(offsets) - 1
    P = int(offsets[-1])
    out = np.full((P, n), np.nan, dtype=np.float64)
    for e in (range(E) if experts is None else experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        w_e = dequant_rows(q_all, np.arange(e * n, (e + 1) * n))
        out[lo:hi] = matmul_f64(a[gather[lo:hi]], w_e)
    return out
