// moe_compact_rows: copy only the rows of a DP-padded buffer that carry data,
// or hand compact rows back to their padded positions.
//
// SGLang PR #6092 (discussion): data-parallel workers of batch sizes such as
// [120, 1, 1, 1, 1, 1, 1, 1] share an FFN input buffer of 8 x 120 rows; only
// each worker's effective rows are copied into the communication buffer, never
// its padding. Block j of the padded buffer (block_rows rows) carries its first
// counts[j] rows; compact row i is the i-th carrying row, block by block.
//
// HBM-bound copy. Every workgroup first forms the exclusive prefix of the
// clamped counts in LDS (at most kMaxPadBlocks of them), so the copy needs no
// host sync. Waves then walk the compact rows with a grid stride: a wave finds
// its row's block by binary search over the prefix (wave-uniform, in LDS),
// loads up to kBatch 1 KiB slabs of the row (64 lanes x 16 bytes, or x 4 bytes
// for rows that are not whole 16-byte vectors) and stores them. Padding rows
// are never visited.
#include "tr_device.h"
#include "tr_internal.h"

namespace tr {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kMaxPadBlocks / kThreads;
constexpr int kBatch = 8;   // slabs loaded before they are stored

template <typename V>
__global__ __launch_bounds__(kThreads) void compact_rows(int64_t T, int B, int nb,
                                                         const int* __restrict__ counts,
                                                         int64_t vpr, const V* __restrict__ src,
                                                         V* __restrict__ dst, int to_padded,
                                                         int* __restrict__ n_out) {
  __shared__ int pre[kMaxPadBlocks + 1];   // block j: compact position of its first row
  __shared__ int tmp[kThreads / kWave];
  const int tid = threadIdx.x;
  // clamped counts, kPerThread consecutive blocks per thread, then the scan.
  // The loads are unconditional (block index clamped; none when T == 0) so
  // that all go out before the first wait; blocks past nb count zero.
  int local[kPerThread];
  if (nb > 0) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) local[u] = counts[min(tid * kPerThread + u, nb - 1)];
  }
  int sum = 0;
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int j = tid * kPerThread + u;
    int c = 0;
    if (j < nb) {
      const int64_t rows = T - static_cast<int64_t>(j) * B;
      const int cap = rows < B ? static_cast<int>(rows) : B;
      c = local[u];
      c = c < 0 ? 0 : (c > cap ? cap : c);
    }
    local[u] = c;
    sum += c;
  }
  int total = 0;
  int run = block_exclusive_scan<kThreads>(sum, tmp, &total);
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int j = tid * kPerThread + u;
    if (j < nb) pre[j] = run;
    run += local[u];
  }
  if (tid == 0) pre[nb] = total;
  if (blockIdx.x == 0 && tid == 0 && n_out) *n_out = total;
  __syncthreads();

  const int lane = lane_id();
  const int64_t gw = __builtin_amdgcn_readfirstlane(
      static_cast<int>((static_cast<int64_t>(blockIdx.x) * kThreads + tid) / kWave));
  const int64_t nw = static_cast<int64_t>(gridDim.x) * (kThreads / kWave);
  for (int64_t c = gw; c < total; c += nw) {
    // the block of compact row c: the last j with pre[j] <= c (blocks that
    // carry nothing share their prefix with the next one, so it carries c)
    int lo = 0, hi = nb - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= c) lo = mid; else hi = mid - 1;
    }
    const int64_t t = static_cast<int64_t>(lo) * B + (c - pre[lo]);
    const V* s = src + (to_padded ? c : t) * vpr;
    V* d = dst + (to_padded ? t : c) * vpr;
    for (int64_t v0 = 0; v0 < vpr; v0 += kBatch * kWave) {
      // loads unconditional (index clamped into the row) so that all go out
      // before the first store waits; stores only in range
      V v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t i = v0 + u * kWave + lane;
        v[u] = s[i < vpr ? i : vpr - 1];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t i = v0 + u * kWave + lane;
        if (i < vpr) d[i] = v[u];
      }
    }
  }
}

template <typename V>
hipError_t launch(int64_t T, int B, const int* counts, int64_t row_bytes, const void* src,
                  void* dst, int to_padded, int* n_out, hipStream_t st) {
  const int64_t vpr = row_bytes / static_cast<int64_t>(sizeof(V));
  const int nb = static_cast<int>(cdiv(T, B));
  int64_t blocks = cdiv(T, kThreads / kWave);   // a wave per row at most
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;          // T == 0 still writes n_out
  hipLaunchKernelGGL(compact_rows<V>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st,
                     T, B, nb, counts, vpr, static_cast<const V*>(src), static_cast<V*>(dst),
                     to_padded, n_out);
  return hipGetLastError();
}

}  // namespace

hipError_t compact_rows(int64_t T, int B, const int* counts, int64_t row_bytes, const void* src,
                        void* dst, bool to_padded, int* n_out, hipStream_t st) {
  const bool vec16 = row_bytes % 16 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(dst) % 16 == 0;
  if (vec16)
    return launch<u32x4>(T, B, counts, row_bytes, src, dst, to_padded, n_out, st);
  return launch<uint32_t>(T, B, counts, row_bytes, src, dst, to_padded, n_out, st);
}

}  // namespace tr
