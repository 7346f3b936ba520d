// probe.hip -- a plain streaming read of a device buffer: the reference
// against which the decode GEMV's HBM rate is judged.  Decode is bound by
// the weight reads ("Low-bit inference for very large MoE", table "Kernels
// on different hardware", row W4A16), so the best rate at which this part
// can read a buffer of the weight's size, with the same rotation past the
// last-level cache, is the ceiling that GEMV can approach; the published 8
// TB/s is a different figure.
//
// Each wave reads eight contiguous 1 KB pieces per iteration (16 bytes per
// lane, non-temporal, all eight in flight), workgroups of 4 waves stride the
// buffer; the values are folded into one word that is written only if it
// equals a constant no buffer of the probe's callers produces, which keeps
// the loads from being removed.  The shape is the best of a sweep on gfx950
// (pieces in flight 4/8/16, plain / non-temporal / global->LDS loads,
// 512..2048 workgroups).
#include "q4_launch.h"
#include "q4_mma.h"

namespace q4 {
namespace {

constexpr int kProbeWaves = 4;
constexpr int kProbeU = 8;
constexpr unsigned kProbeGrid = 1024;
constexpr uint32_t kProbeMagic = 0x9E3779B9u;

__global__ void __launch_bounds__(kProbeWaves * 64)
read_probe_kernel(const uint8_t* __restrict__ p, int64_t nchunks, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nw = (int64_t)gridDim.x * kProbeWaves;
  u32x4_t acc = u32x4_t{0u, 0u, 0u, 0u};
  int64_t c = ((int64_t)blockIdx.x * kProbeWaves + wave) * kProbeU;
  for (; c + kProbeU <= nchunks; c += nw * kProbeU) {
    u32x4_t v[kProbeU];
#pragma unroll
    for (int u = 0; u < kProbeU; ++u)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + (c + u) * 1024 + lane * 16));
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) acc ^= v[u];
  }
  for (; c < nchunks; ++c)  // the last wave's partial group of pieces
    acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + c * 1024 + lane * 16));
  const uint32_t w = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (w == kProbeMagic) sink[0] = w;
}

}  // namespace

hipError_t launch_read_probe(const uint8_t* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t nchunks = bytes / 1024;
  if (nchunks == 0) return hipSuccess;
  const int64_t need = (nchunks + kProbeU * kProbeWaves - 1) / (kProbeU * kProbeWaves);
  const unsigned grid = (unsigned)(need < kProbeGrid ? need : kProbeGrid);
  read_probe_kernel<<<grid, kProbeWaves * 64, 0, stream>>>(src, nchunks, sink);
  return hipGetLastError();
}

}  // namespace q4
