// Device-side helpers shared by the libtopreduce kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tr {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 <-> fp32. Widening is exact (bf16 is the top half of an fp32);
// narrowing rounds to nearest even and keeps NaN a quiet NaN.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// Two floats into one dword of two bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Count of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ int popc_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

// Exclusive prefix sum over the threads of a block of `kThreads` (multiple of
// 64). `tmp` is LDS of kThreads/64 ints. Returns the prefix; *total gets the
// block sum. Ends with a barrier, so `tmp` can be reused right after.
template <int kThreads>
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  constexpr int kWaves = kThreads / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) tmp[wave] = incl;
  __syncthreads();
  int wave_base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    int t = tmp[w];
    if (w < wave) wave_base += t;
    sum += t;
  }
  __syncthreads();
  *total = sum;
  return wave_base + incl - v;
}

// Integer ceil-div.
__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace tr
