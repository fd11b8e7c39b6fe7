// moe_combine_reduce: weighted top-k reduce back into received order,
//   y[t] = sum over k ascending with row_map[t][k] >= 0 of w[t][k] * O[row_map[t][k]]
// accumulated in fp32 and rounded once (nearest even) to the output type; a
// row without a local slot is written as +0.
//
// DeepEP issue #48 answer: the reduction before the combine all-to-all.
// DeepEP issue #760: the combine epilogue assigns one warp per output token and
// straggles when a rank holds only a handful of tokens. Here the unit of work
// is a wavefront-sized slab of one token's row (64 lanes x 8 elements), so a
// single token still spreads over H/512 wavefronts on as many CUs, and with
// many tokens the same grid streams O at HBM rate. The token of a slab is
// wave-uniform: its row_map and weight entries are scalar loads, and the
// loads of up to 8 slots are issued before they are summed in slot order.
// Weights of non-local slots are never read.
#include "tr_device.h"
#include "tr_internal.h"

namespace tr {
namespace {

constexpr int kThreads = 256;
constexpr int kSlab = kWave * 8;  // elements per wave item
constexpr int kBatch = 8;         // slots loaded before accumulating (16 and 32 measured slower)

template <bool kBF16>
struct Row8;

template <>
struct Row8<true> {
  u32x4 v;
  __device__ __forceinline__ void load(const void* base, int64_t off) {
    v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off);
  }
  __device__ __forceinline__ void zero() { v = u32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = v[i >> 1];
    return bf16_bits_to_f32((i & 1) ? (w >> 16) : (w & 0xffffu));
  }
  static __device__ __forceinline__ void store(void* base, int64_t off, const float* a) {
    u32x4 o;
    o[0] = pack_bf16x2(a[0], a[1]);
    o[1] = pack_bf16x2(a[2], a[3]);
    o[2] = pack_bf16x2(a[4], a[5]);
    o[3] = pack_bf16x2(a[6], a[7]);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + off) = o;
  }
};

template <>
struct Row8<false> {
  u32x4 v0, v1;
  __device__ __forceinline__ void load(const void* base, int64_t off) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + off);
    v0 = p[0];
    v1 = p[1];
  }
  __device__ __forceinline__ void zero() { v0 = v1 = u32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ float get(int i) const {
    return __uint_as_float(i < 4 ? v0[i] : v1[i - 4]);
  }
  static __device__ __forceinline__ void store(void* base, int64_t off, const float* a) {
    u32x4* p = reinterpret_cast<u32x4*>(static_cast<float*>(base) + off);
    p[0] = u32x4{__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
                 __float_as_uint(a[3])};
    p[1] = u32x4{__float_as_uint(a[4]), __float_as_uint(a[5]), __float_as_uint(a[6]),
                 __float_as_uint(a[7])};
  }
};

// Rows at or past n_rows count as absent, like -1. With `rest`, only the
// tokens rest[0 .. *rest_n) are written (the others have exactly one local
// slot, and GEMM2 has written them).
template <bool kBF16>
__global__ __launch_bounds__(kThreads) void combine_rows(const void* __restrict__ O,
                                                         const int* __restrict__ row_map,
                                                         const float* __restrict__ w, int64_t T,
                                                         int K, int64_t H, int64_t n_rows,
                                                         const int* __restrict__ rest,
                                                         const int* __restrict__ rest_n,
                                                         void* __restrict__ y) {
  const int64_t nslab = (H + kSlab - 1) / kSlab;
  const int lane = lane_id();
  const int64_t gw = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * (kThreads / kWave);
  // y[t] over the slab of columns starting at col (this lane: col .. col + 7)
  auto reduce_slab = [&](int64_t t, int64_t col) {
    const bool active = col < H;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int k0 = 0; k0 < K; k0 += kBatch) {
      int rows[kBatch];
      float wk[kBatch];
      Row8<kBF16> v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int k = k0 + j;
        rows[j] = k < K ? row_map[t * K + k] : -1;
        if (rows[j] >= n_rows) rows[j] = -1;
        wk[j] = 0.0f;
        v[j].zero();
        if (rows[j] >= 0) {
          wk[j] = w ? w[t * K + k] : 1.0f;
          if (active) v[j].load(O, static_cast<int64_t>(rows[j]) * H + col);
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (rows[j] >= 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(wk[j], v[j].get(i), acc[i]);
        }
    }
    if (active) Row8<kBF16>::store(y, t * H + col, acc);
  };
  const int64_t ntok = rest ? *rest_n : T;
  const int64_t items = ntok * nslab;
  for (int64_t item = gw; item < items; item += nw) {
    const int64_t q = __builtin_amdgcn_readfirstlane(static_cast<int>(item / nslab));
    const int64_t t = rest ? rest[q] : q;
    reduce_slab(t, (item - q * nslab) * kSlab + static_cast<int64_t>(lane) * 8);
  }
}

}  // namespace

namespace {

hipError_t launch_rows(bool bf16, const void* O, const int* row_map, const float* w, int64_t T,
                       int K, int64_t H, int64_t n_rows, const int* rest, const int* rest_n,
                       void* y, hipStream_t st) {
  const int64_t nslab = (H + kSlab - 1) / kSlab;
  const int64_t waves = T * nslab;
  int64_t blocks = cdiv(waves, kThreads / kWave);
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 32;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(combine_rows<true>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       st, O, row_map, w, T, K, H, n_rows, rest, rest_n, y);
  else
    hipLaunchKernelGGL(combine_rows<false>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       st, O, row_map, w, T, K, H, n_rows, rest, rest_n, y);
  return hipGetLastError();
}

}  // namespace

hipError_t combine_reduce(const tr_moe_plan& p, const void* expert_out, const float* w, void* y,
                          hipStream_t st, bool skip_single) {
  const tr_moe_desc& d = p.d;
  const void* O = expert_out ? expert_out : p.O;
  return launch_rows(d.dtype == TR_BF16, O, p.row_map, w, d.T, d.K, d.H, p.R_cap,
                     skip_single ? p.tok_rest : nullptr, skip_single ? p.stats + 4 : nullptr, y,
                     st);
}

// The cross-rank epilogue is the same reduction with unit weights over the
// caller's index map: one wavefront per 512-element slab of an output row, so
// a handful of tokens still spreads over many wavefronts (DeepEP issue #760,
// the first proposed fix).
hipError_t combine_epilogue(int64_t T, int J, int64_t H, bool bf16, const int* src,
                            const void* recv, int64_t n_recv, void* y, hipStream_t st) {
  return launch_rows(bf16, recv, src, nullptr, T, J, H, n_recv, nullptr, nullptr, y, st);
}

}  // namespace tr
