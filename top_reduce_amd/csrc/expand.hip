// moe_expand: copy each received row once per local route into the
// expert-contiguous buffer, Xe[r] = x[row_src[r]] (DeepEP issue #48 answer:
// with a grouped GEMM one token must be expanded to several experts).
//
// HBM-bound row gather. The number of rows R lives on the device
// (offsets[E]); the grid is sized for the upper bound and every wave walks
// 1 KiB slabs (64 lanes x 16 bytes) of rows with a grid stride, so there is
// no host sync and no per-row launch cost. The source row index is
// wave-uniform (scalar load); each wave keeps kUnroll 16-byte loads in
// flight before storing.
#include "tr_device.h"
#include "tr_internal.h"

namespace tr {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void expand_rows(const u32x4* __restrict__ x,
                                                        const int* __restrict__ row_src,
                                                        const int* __restrict__ R_ptr,
                                                        int64_t chunks, u32x4* __restrict__ Xe) {
  const int64_t R = *R_ptr;
  const int64_t nslab = (chunks + kWave - 1) / kWave;
  const int64_t items = R * nslab;
  const int lane = lane_id();
  const int64_t gw = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * (kThreads / kWave);
  for (int64_t it = gw * kUnroll; it < items; it += nw * kUnroll) {
    u32x4 v[kUnroll];
    int64_t dst[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      dst[u] = -1;
      const int64_t item = it + u;
      if (item < items) {
        const int r = __builtin_amdgcn_readfirstlane(static_cast<int>(item / nslab));
        const int64_t c = (item - static_cast<int64_t>(r) * nslab) * kWave + lane;
        const int src = row_src[r];
        if (c < chunks) {
          v[u] = x[static_cast<int64_t>(src) * chunks + c];
          dst[u] = static_cast<int64_t>(r) * chunks + c;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (dst[u] >= 0) Xe[dst[u]] = v[u];
  }
}

}  // namespace

hipError_t expand(const tr_moe_plan& p, const void* x, hipStream_t st) {
  const int64_t es = p.d.dtype == TR_BF16 ? 2 : 4;
  const int64_t chunks = p.d.H * es / 16;
  const int64_t nslab = (chunks + kWave - 1) / kWave;
  const int64_t waves = cdiv(p.R_cap * nslab, kUnroll);
  int64_t blocks = cdiv(waves, kThreads / kWave);
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 16;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(expand_rows, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st,
                     static_cast<const u32x4*>(x), p.row_src, p.offsets + p.d.E, chunks,
                     static_cast<u32x4*>(p.Xe));
  return hipGetLastError();
}

}  // namespace tr
