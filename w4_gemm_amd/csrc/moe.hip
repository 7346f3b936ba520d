// moe.hip -- the steps of an MoE layer around the grouped expert GEMM:
// routing (top-k experts per token with softmax gates, then a stable
// expert-major dispatch order), the SwiGLU activation between the gate/up
// and down expert GEMMs, and the gated combine of each token's expert
// outputs.  The grouped GEMMs themselves are grouped.hip / gemm.hip.
//
// "Low-bit inference for very large MoE", "A few details": one low-bit
// weight matrix per expert, the tokens grouped by routing.  Readings where
// the pages are silent: a token's experts are its k largest router logits
// (ties to the lower expert id), its gate for each is that expert's softmax
// probability over all E logits (fp32, not renormalized); routed rows are
// ordered expert-major, tokens ascending within an expert; the expert FFN is
// SwiGLU, h = silu(gate) * up, silu(z) = z / (1 + exp(-z)).
#include "q4_device.h"
#include "q4_launch.h"

namespace q4 {
namespace {

constexpr int kMaxLogitsPerLane = 16;  // E <= 1024 = 16 per lane of one wave
constexpr int kRouteWaves = 4;

// Logits are ordered by integer keys that order floats as their values do
// (-0 folded into +0; NaN above +inf when its sign is clear, below -inf
// otherwise), so that NaN logits still leave a strict order in which every
// chosen expert is a distinct valid one.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// One wave per token: softmax statistics over the E logits, then k rounds
// of a wave-wide argmax (largest key, ties to the lower expert id).
__global__ void __launch_bounds__(64 * kRouteWaves)
moe_topk_kernel(const float* __restrict__ logits, int64_t ld, int T, int E, int k,
                int32_t* __restrict__ ids, float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (int64_t)t * ld;
  float v[kMaxLogitsPerLane];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxLogitsPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -INFINITY;
    m = fmaxf(m, v[i]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxLogitsPerLane; ++i)
    if (lane + 64 * i < E) s += expf(v[i] - m);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  uint32_t used = 0;
  for (int j = 0; j < k; ++j) {
    // the lane's best remaining logit (lowest expert id on ties; a lane with
    // none left keeps key 0 and id INT_MAX, below every valid candidate)
    uint32_t bk = 0u;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxLogitsPerLane; ++i) {
      const int e = lane + 64 * i;
      const uint32_t ki = order_key(v[i]);
      if (e < E && !((used >> i) & 1u) && (ki > bk || (ki == bk && e < be))) {
        bk = ki;
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t ok = __shfl_xor(bk, off);
      const int oe = __shfl_xor(be, off);
      if (ok > bk || (ok == bk && oe < be)) {
        bk = ok;
        be = oe;
      }
    }
    if ((be & 63) == lane) used |= 1u << (be >> 6);
    if (lane == 0) {
      ids[(int64_t)t * k + j] = be;
      weights[(int64_t)t * k + j] = expf(key_value(bk) - m) / s;
    }
  }
}

// E <= 64: one logit per lane, and each chosen expert's slot is its rank
// among the token's logits in the same order (larger key first, the lower
// expert id on ties), counted against the keys copied to LDS -- one pass
// instead of k rounds of a wave-wide argmax.  The ranks are a permutation,
// so each of the k slots is written exactly once.  The softmax statistics
// are reduced as above (same order, same bits).
__global__ void __launch_bounds__(64 * kRouteWaves)
moe_topk64_kernel(const float* __restrict__ logits, int64_t ld, int T, int E, int k,
                  int32_t* __restrict__ ids, float* __restrict__ weights) {
  __shared__ __attribute__((aligned(16))) uint32_t keys[kRouteWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x * kRouteWaves + w;
  if (t >= T) return;                      // (whole waves: no barrier below)
  const bool valid = lane < E;
  const float v = valid ? logits[(int64_t)t * ld + lane] : -INFINITY;
  float m = fmaxf(-INFINITY, v);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float s = valid ? expf(v - m) : 0.0f;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  // lanes past E hold the smallest key; their ids are above every valid one,
  // so they never rank ahead of a valid lane
  const uint32_t key = valid ? order_key(v) : 0u;
  keys[w][lane] = key;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int rank = 0;
#pragma unroll
  for (int j = 0; j < 64; j += 4) {
    const uint4 q = *reinterpret_cast<const uint4*>(&keys[w][j]);
    rank += (q.x > key || (q.x == key && j < lane)) + (q.y > key || (q.y == key && j + 1 < lane)) +
            (q.z > key || (q.z == key && j + 2 < lane)) + (q.w > key || (q.w == key && j + 3 < lane));
  }
  if (valid && rank < k) {
    ids[(int64_t)t * k + rank] = lane;
    weights[(int64_t)t * k + rank] = expf(v - m) / s;
  }
}

constexpr int kDispatchThreads = 1024;

// One workgroup: per-expert counts and a token bitmap per expert in LDS, the
// expert offsets (exclusive scan), then each choice's row = offset of its
// expert + number of earlier tokens routed to that expert.
__global__ void __launch_bounds__(kDispatchThreads)
moe_dispatch_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                    int32_t* __restrict__ offsets, int32_t* __restrict__ gather,
                    int32_t* __restrict__ inv) {
  extern __shared__ uint32_t lds[];
  const int W = (T + 31) >> 5;             // bitmap words per expert
  uint32_t* counts = lds;                  // [E]
  uint32_t* offs = lds + E;                // [E]
  uint32_t* bits = lds + 2 * E;            // [E][W]
  uint32_t* pre = bits + (size_t)E * W;    // [E][W] set bits in earlier words
  const int tid = threadIdx.x;
  const int64_t P = (int64_t)T * k;
  for (int64_t i = tid; i < (int64_t)E * W; i += kDispatchThreads) bits[i] = 0u;
  for (int e = tid; e < E; e += kDispatchThreads) counts[e] = 0u;
  __syncthreads();
  for (int64_t i = tid; i < P; i += kDispatchThreads) {
    const int t = (int)(i / k), e = ids[i];
    atomicOr(&bits[(size_t)e * W + (t >> 5)], 1u << (t & 31));
    atomicAdd(&counts[e], 1u);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kDispatchThreads) {
    uint32_t run = 0;
    for (int w = 0; w < W; ++w) {
      pre[(size_t)e * W + w] = run;
      run += __popc(bits[(size_t)e * W + w]);
    }
  }
  // expert offsets: exclusive scan of the counts by wave 0 alone (E <= 1024:
  // lane l sums experts 16l .. 16l + 15, then a scan across the lanes)
  if (tid < 64) {
    const int e0 = tid * 16;
    uint32_t c[16], sum = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      c[i] = e0 + i < E ? counts[e0 + i] : 0u;
      sum += c[i];
    }
    uint32_t x = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(x, off);
      if (tid >= off) x += y;
    }
    uint32_t run = x - sum;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (e0 + i < E) {
        offs[e0 + i] = run;
        offsets[e0 + i] = (int32_t)run;
      }
      run += c[i];
    }
    if (tid == 63) offsets[E] = (int32_t)x;
  }
  __syncthreads();
  for (int64_t i = tid; i < P; i += kDispatchThreads) {
    const int t = (int)(i / k), e = ids[i];
    const size_t wi = (size_t)e * W + (t >> 5);
    const uint32_t rank = pre[wi] + __popc(bits[wi] & ((1u << (t & 31)) - 1u));
    const int32_t pos = (int32_t)(offs[e] + rank);
    gather[pos] = t;
    inv[i] = pos;
  }
}

constexpr int kThreads = 256;

// h[p][n] = bf16(silu(gu[p][n]) * gu[p][I + n]), 8 values per thread.
__global__ void __launch_bounds__(kThreads)
swiglu_kernel(const uint16_t* __restrict__ gu, int64_t ld_gu, int64_t P, int64_t I,
              uint16_t* __restrict__ h, int64_t ldh) {
  const int64_t cpr = I >> 3, total = P * cpr;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * kThreads) {
    const int64_t p = c / cpr, n0 = (c - p * cpr) * 8;
    const uint4 g = *reinterpret_cast<const uint4*>(gu + p * ld_gu + n0);
    const uint4 u = *reinterpret_cast<const uint4*>(gu + p * ld_gu + I + n0);
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float g0 = bf16_lo(gw[j]), g1 = bf16_hi(gw[j]);
      const float a0 = g0 / (1.0f + expf(-g0)) * bf16_lo(uw[j]);
      const float a1 = g1 / (1.0f + expf(-g1)) * bf16_hi(uw[j]);
      o[j] = f32_to_bf16_rne(a0) | (f32_to_bf16_rne(a1) << 16);
    }
    *reinterpret_cast<uint4*>(h + p * ldh + n0) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// out[t][n] = bf16(sum_j w[t][j] * y[inv[t][j]][n]), fp32 in choice order;
// one workgroup per (token, 2048-column slice), 8 columns per thread.
__global__ void __launch_bounds__(kThreads)
moe_combine_kernel(const uint16_t* __restrict__ y, int64_t ldy, const int32_t* __restrict__ inv,
                   const float* __restrict__ w, int k, int64_t N, uint16_t* __restrict__ out,
                   int64_t ldo) {
  const int64_t slices = (N + kThreads * 8 - 1) / (kThreads * 8);
  const int64_t t = blockIdx.x / slices;
  const int64_t n0 = ((int64_t)(blockIdx.x % slices) * kThreads + threadIdx.x) * 8;
  if (n0 >= N) return;
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int j = 0; j < k; ++j) {
    const int64_t p = inv[t * k + j];
    const float g = w[t * k + j];
    const uint4 v = *reinterpret_cast<const uint4*>(y + p * ldy + n0);
    const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = __builtin_fmaf(g, bf16_lo(vw[q]), acc[2 * q]);
      acc[2 * q + 1] = __builtin_fmaf(g, bf16_hi(vw[q]), acc[2 * q + 1]);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = f32_to_bf16_rne(acc[2 * q]) | (f32_to_bf16_rne(acc[2 * q + 1]) << 16);
  *reinterpret_cast<uint4*>(out + t * ldo + n0) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

size_t moe_dispatch_lds_bytes(int64_t T, int32_t E) {
  return (size_t)4 * (2 * (size_t)E + 2 * (size_t)E * (size_t)((T + 31) / 32));
}

hipError_t launch_moe_route(const float* logits, int64_t ld, int64_t T, int32_t E, int32_t k,
                            int32_t* ids, float* weights, int32_t* offsets, int32_t* gather,
                            int32_t* inv, hipStream_t stream) {
  if (T > 0) {
    const unsigned grid = (unsigned)((T + kRouteWaves - 1) / kRouteWaves);
    if (E <= 64)
      moe_topk64_kernel<<<grid, 64 * kRouteWaves, 0, stream>>>(logits, ld, (int)T, E, k, ids, weights);
    else
      moe_topk_kernel<<<grid, 64 * kRouteWaves, 0, stream>>>(logits, ld, (int)T, E, k, ids, weights);
  }
  const size_t lds = moe_dispatch_lds_bytes(T, E);
  const hipError_t attr = set_max_lds<&moe_dispatch_kernel>(kMoeDispatchMaxLds);
  if (attr != hipSuccess) return attr;
  moe_dispatch_kernel<<<1, kDispatchThreads, lds, stream>>>(ids, (int)T, E, k, offsets, gather, inv);
  return hipGetLastError();
}

hipError_t launch_swiglu(const uint16_t* gu, int64_t ld_gu, int64_t P, int64_t I, uint16_t* h, int64_t ldh,
                         hipStream_t stream) {
  const int64_t chunks = P * (I >> 3);
  if (!chunks) return hipSuccess;
  int64_t b = (chunks + kThreads - 1) / kThreads;
  if (b > (1 << 20)) b = 1 << 20;
  swiglu_kernel<<<(unsigned)b, kThreads, 0, stream>>>(gu, ld_gu, P, I, h, ldh);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t* y, int64_t ldy, const int32_t* inv, const float* w, int64_t T,
                              int32_t k, int64_t N, uint16_t* out, int64_t ldo, hipStream_t stream) {
  if (T == 0 || N == 0) return hipSuccess;
  const unsigned grid = (unsigned)(T * ((N + kThreads * 8 - 1) / (kThreads * 8)));
  moe_combine_kernel<<<grid, kThreads, 0, stream>>>(y, ldy, inv, w, k, N, out, ldo);
  return hipGetLastError();
}

}  // namespace q4
