"""Seeded synthetic inputs for the quantize / W4 matmul workloads.

This module only draws random numbers and arranges them; it holds none of
the quantization or matmul arithmetic, so the HIP path and the CPU oracle can
both be fed from it.

Recipe (the same for every workload):
  * standard normals are drawn in fp32 from numpy's PCG64, in chunks of 2^22
    values; chunk i of a named stream uses SeedSequence(seed, spawn_key=
    (crc32(name), i)), so the values do not depend on how many threads fill
    them;
  * they are multiplied by the stated std in fp32, outlier entries (or
    channels) are multiplied by their factor in fp32, and the result is
    rounded once to bf16 (round to nearest even);
  * outlier positions are round(frac * count) distinct indices drawn with
    Generator.choice(replace=False) from the stream "<name>/outliers".

The five workloads are those of the benchmark: a small INT4 g128 GEMV, the
MXFP4 decode GEMV (28672x8192), the NVFP4 prefill GEMM (4096x8192x8192), the
MoE grouped expert GEMM (64 experts of 2048x7168, 256 tokens, top-8), the
W4A4 MXFP4 GEMM (8192^3) and the W4A8 GEMM (INT4 weights, per-token FP8
activations, 4096x8192x8192).
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK = 1 << 22


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _seedseq(seed: int, name: str, *extra: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(seed, spawn_key=(zlib.crc32(name.encode()), *extra))


def normal_f32(name: str, n: int, seed: int = 0) -> np.ndarray:
    """n standard normals (fp32) of the named stream."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(i):
        g = np.random.Generator(np.random.PCG64(_seedseq(seed, name, i)))
        lo = i * CHUNK
        g.standard_normal(out=out[lo:min(n, lo + CHUNK)], dtype=np.float32)

    if nchunks <= 1:
        if n:
            fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def choose(name: str, population: int, count: int, seed: int = 0) -> np.ndarray:
    """`count` distinct indices in [0, population), sorted."""
    g = np.random.Generator(np.random.PCG64(_seedseq(seed, name + "/outliers")))
    return np.sort(g.choice(population, size=count, replace=False))


def normal_f32_range(name: str, lo: int, hi: int, seed: int = 0) -> np.ndarray:
    """Values [lo, hi) of the named stream (the same numbers normal_f32
    gives at those positions), generating only the chunks that cover them."""
    c0, c1 = lo // CHUNK, (hi + CHUNK - 1) // CHUNK
    out = np.empty((c1 - c0) * CHUNK, dtype=np.float32)
    for i in range(c0, c1):
        g = np.random.Generator(np.random.PCG64(_seedseq(seed, name, i)))
        g.standard_normal(out=out[(i - c0) * CHUNK:(i - c0 + 1) * CHUNK], dtype=np.float32)
    return out[lo - c0 * CHUNK:hi - c0 * CHUNK]


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """fp32 -> bf16 (round to nearest even), as a CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def matrix(name: str, rows: int, cols: int, std: float, seed: int = 0,
           outlier_frac: float = 0.0, outlier_mult: float = 1.0,
           channel_frac: float = 0.0, channel_mult: float = 1.0) -> torch.Tensor:
    """bf16 [rows, cols] ~ N(0, std^2), with optional entry outliers
    (a fraction of all entries multiplied by outlier_mult) or channel
    outliers (a fraction of the columns multiplied by channel_mult)."""
    x = normal_f32(name, rows * cols, seed)
    x *= np.float32(std)
    if outlier_frac:
        cnt = int(round(outlier_frac * rows * cols))
        idx = choose(name, rows * cols, cnt, seed)
        x[idx] *= np.float32(outlier_mult)
    x = x.reshape(rows, cols)
    if channel_frac:
        cnt = int(round(channel_frac * cols))
        ch = choose(name, cols, cnt, seed)
        x[:, ch] *= np.float32(channel_mult)
    return to_bf16(x)


def matrix_rows(name: str, rows: int, cols: int, std: float, r0: int, r1: int,
                seed: int = 0) -> torch.Tensor:
    """Rows [r0, r1) of matrix(name, rows, cols, std, seed) (no outliers)."""
    assert 0 <= r0 <= r1 <= rows
    x = normal_f32_range(name, r0 * cols, r1 * cols, seed) * np.float32(std)
    return to_bf16(x.reshape(r1 - r0, cols))


@dataclass
class Routing:
    """Top-k routing of tokens to experts, rows grouped expert-major."""
    gather: np.ndarray        # int32 [P]: token of each routed row
    offsets: np.ndarray       # int32 [E+1]: rows of expert e are [offsets[e], offsets[e+1])
    topk_ids: np.ndarray      # int64 [T, k]


def route(logits: np.ndarray, k: int) -> Routing:
    """Top-k experts per token by logit (ties to the lower expert id), then a
    counting sort of the (token, expert) pairs by expert, tokens ascending."""
    T, E = logits.shape
    order = np.argsort(-logits, axis=1, kind="stable")
    topk = order[:, :k]
    counts = np.bincount(topk.ravel(), minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    gather = np.empty(T * k, dtype=np.int32)
    fill = offsets[:-1].copy()
    for t in range(T):
        for e in topk[t]:
            gather[fill[e]] = t
            fill[e] += 1
    return Routing(gather, offsets.astype(np.int32), topk)


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    fmt: str
    tensors: dict = field(default_factory=dict)
    meta: dict = field(default_factory=dict)


def int4_gemv(seed: int = 0, n: int = 1024, k: int = 1024, batch: int = 1) -> Workload:
    """INT4 g128: W ~ N(0, 0.02^2) with 0.1% of entries x20; x ~ N(0, 1)."""
    w = matrix("int4_gemv/W", n, k, 0.02, seed, outlier_frac=0.001, outlier_mult=20.0)
    x = matrix("int4_gemv/x", batch, k, 1.0, seed)
    return Workload("int4_g128_gemv", "int4", {"W": w, "x": x}, {"N": n, "K": k, "B": batch})


def mxfp4_gemv(seed: int = 0, n: int = 28672, k: int = 8192, batches=(1, 4, 16)) -> Workload:
    """MXFP4 decode: W ~ N(0, 0.015^2) with 0.05% of entries x30; x ~ N(0, 1)."""
    w = matrix("mxfp4_gemv/W", n, k, 0.015, seed, outlier_frac=0.0005, outlier_mult=30.0)
    xs = {b: matrix(f"mxfp4_gemv/x{b}", b, k, 1.0, seed) for b in batches}
    t = {"W": w}
    t.update({f"x{b}": xs[b] for b in batches})
    return Workload("mxfp4_decode_gemv", "mxfp4", t, {"N": n, "K": k, "batches": tuple(batches)})


def nvfp4_gemm(seed: int = 0, m: int = 4096, n: int = 8192, k: int = 8192) -> Workload:
    """NVFP4 prefill: A ~ N(0, 1) with 1% of channels x10; W ~ N(0, 0.02^2)."""
    a = matrix("nvfp4_gemm/A", m, k, 1.0, seed, channel_frac=0.01, channel_mult=10.0)
    w = matrix("nvfp4_gemm/W", n, k, 0.02, seed)
    return Workload("nvfp4_w4a16_gemm", "nvfp4", {"A": a, "W": w}, {"M": m, "N": n, "K": k})


def moe_grouped(seed: int = 0, experts: int = 64, n: int = 2048, k: int = 7168,
                tokens: int = 256, topk: int = 8) -> Workload:
    """MoE: per-expert W_up [n, k] ~ N(0, 0.02^2) (expert-major rows),
    A ~ N(0, 1), logits [tokens, experts] ~ N(0, 1) -> top-k routing."""
    w = matrix("moe/W", experts * n, k, 0.02, seed)
    a = matrix("moe/A", tokens, k, 1.0, seed)
    logits = normal_f32("moe/logits", tokens * experts, seed).reshape(tokens, experts)
    r = route(logits, topk)
    return Workload("moe_grouped_mxfp4", "mxfp4", {"W": w, "A": a},
                    {"E": experts, "N": n, "K": k, "T": tokens, "topk": topk,
                     "routing": r, "logits": logits})


def w4a8_gemm(seed: int = 0, m: int = 4096, n: int = 8192, k: int = 8192) -> Workload:
    """W4A8 prefill, the prefill shape: A ~ N(0, 1) with 1% of channels x10
    (per-token FP8), W ~ N(0, 0.02^2) (INT4 g128)."""
    a = matrix("w4a8/A", m, k, 1.0, seed, channel_frac=0.01, channel_mult=10.0)
    w = matrix("w4a8/W", n, k, 0.02, seed)
    return Workload("w4a8_int4_fp8_gemm", "int4", {"A": a, "W": w}, {"M": m, "N": n, "K": k})


def moe_layer(seed: int = 0, experts: int = 64, inter: int = 2048, hidden: int = 7168,
              tokens: int = 256, topk: int = 8) -> Workload:
    """MoE FFN layer around the grouped GEMM, the MoE workload's shapes:
    x [tokens, hidden] and router logits [tokens, experts] are the MoE
    workload's A and logits; per expert e, W_up_e is rows [e*inter, (e+1)*
    inter) of its W, W_gate_e the same rows of the stream "moe/Wgate" and
    W_down_e rows [e*hidden, (e+1)*hidden) of "moe/Wdown" [experts*hidden,
    inter], all ~ N(0, 0.02^2).  `expert(e)` returns (W_gu_e = [W_gate_e;
    W_up_e] bf16 [2*inter, hidden], W_down_e bf16 [hidden, inter]) without
    generating the other experts."""
    a = matrix("moe/A", tokens, hidden, 1.0, seed)
    logits = normal_f32("moe/logits", tokens * experts, seed).reshape(tokens, experts)

    def expert(e):
        up = matrix_rows("moe/W", experts * inter, hidden, 0.02, e * inter, (e + 1) * inter, seed)
        gate = matrix_rows("moe/Wgate", experts * inter, hidden, 0.02, e * inter, (e + 1) * inter, seed)
        down = matrix_rows("moe/Wdown", experts * hidden, inter, 0.02, e * hidden, (e + 1) * hidden, seed)
        return torch.cat([gate, up]), down

    return Workload("moe_layer_mxfp4", "mxfp4", {"x": a},
                    {"E": experts, "I": inter, "K": hidden, "T": tokens, "topk": topk,
                     "logits": logits, "expert": expert})


def w4a4_gemm(seed: int = 0, m: int = 8192, n: int = 8192, k: int = 8192) -> Workload:
    """W4A4 MXFP4: A ~ N(0, 1), W ~ N(0, 0.02^2), both quantized along K."""
    a = matrix("w4a4/A", m, k, 1.0, seed)
    w = matrix("w4a4/W", n, k, 0.02, seed)
    return Workload("w4a4_mxfp4_gemm", "mxfp4", {"A": a, "W": w}, {"M": m, "N": n, "K": k})
