// moe_expand: copy each received row once per local route into the
// expert-contiguous buffer, Xe[row_map[t, k]] = x[t] (DeepEP issue #48 answer:
// with a grouped GEMM one token must be expanded to several experts).
//
// HBM-bound scatter in received order. A wave owns one token at a time: it
// reads the token's slot map (scalar loads), skips the token if no slot is
// local (padding rows cost one map read), loads up to kBatch 1 KiB slabs of
// the row (64 lanes x 16 bytes) and stores them to every local slot's row.
// Each input row is read from HBM once however many local experts it has;
// rows are walked with a grid stride, so there is no host sync.
#include "tr_device.h"
#include "tr_internal.h"

namespace tr {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;

__global__ __launch_bounds__(kThreads) void expand_rows(const u32x4* __restrict__ x,
                                                        const int* __restrict__ row_map, int64_t T,
                                                        int K, int64_t chunks,
                                                        u32x4* __restrict__ Xe) {
  const int lane = lane_id();
  const int64_t gw = __builtin_amdgcn_readfirstlane(
      static_cast<int>((static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave));
  const int64_t nw = static_cast<int64_t>(gridDim.x) * (kThreads / kWave);
  for (int64_t t = gw; t < T; t += nw) {
    const int* rm = row_map + t * K;
    bool any = false;
    for (int k = 0; k < K; ++k) any |= rm[k] >= 0;
    if (!any) continue;
    const u32x4* src = x + t * chunks;
    for (int64_t c0 = 0; c0 < chunks; c0 += kBatch * kWave) {
      u32x4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t c = c0 + u * kWave + lane;
        if (c < chunks) v[u] = src[c];
      }
      for (int k = 0; k < K; ++k) {
        const int r = rm[k];
        if (r < 0) continue;
        u32x4* dst = Xe + static_cast<int64_t>(r) * chunks;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int64_t c = c0 + u * kWave + lane;
          if (c < chunks) dst[c] = v[u];
        }
      }
    }
  }
}

}  // namespace

hipError_t expand(const tr_moe_plan& p, const void* x, hipStream_t st) {
  const int64_t es = p.d.dtype == TR_BF16 ? 2 : 4;
  const int64_t chunks = p.d.H * es / 16;
  int64_t blocks = cdiv(p.d.T, kThreads / kWave);
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(expand_rows, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st,
                     static_cast<const u32x4*>(x), p.row_map, p.d.T, p.d.K, chunks,
                     static_cast<u32x4*>(p.Xe));
  return hipGetLastError();
}

}  // namespace tr
