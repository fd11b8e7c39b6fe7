// moe_grouped_gemm: the local experts' SwiGLU MLP over the expert-contiguous
// rows Xe (DeepEP issue #48 answer: a grouped GEMM over expanded tokens).
//
//   GEMM1 + SwiGLU: h[r, i] = silu(Xe[r] . W1[e][i]) * (Xe[r] . W1[e][I + i])
//   GEMM2:          O[r, j] = h[r] . W2[e][j]
// for every expanded row r of expert e's segment. Both GEMMs are "NT": the
// activation rows and the weight rows are contiguous along the reduction
// dimension. Accumulation is fp32; h and O are rounded once to the storage
// type.
//
// Work is scheduled on the device from counts/offsets, never from the host:
// empty experts and rows past each segment have no tile at all (SGLang PR
// #6092: zero-length padded rows of a DP global batch must not add GEMM
// work). Two bf16 kernels share the experts:
//
//  - gemm_tiled: persistent 256x256x64 block tiles on bf16 MFMA
//    (v_mfma_f32_32x32x16_bf16), four waves each owning a 128x128 quadrant,
//    operands staged through XOR-swizzled LDS with a register prefetch of the
//    next k-tile. Tiles are numbered expert-major with groups of 4 m-tiles and
//    handed to the 8 XCDs in contiguous chunks so that concurrent tiles of an
//    XCD share A and B tiles in its L2. For GEMM1 each B tile holds 128 gate
//    rows and the matching 128 up rows, so a lane owns gate and up of the
//    same outputs and SwiGLU runs in the epilogue.
//  - gemm_stream: experts with few rows (decode). Weight rows are streamed
//    once from HBM straight into the A operand of v_mfma_f32_16x16x32_bf16;
//    up to 32 token rows ride in the B operand; the reduction dimension is
//    split over the four waves of a block and summed in LDS in a fixed order.
//
// An fp32 variant (gemm_f32) covers fp32 inputs with plain fp32 FMAs.
#include "tr_device.h"
#include "tr_internal.h"

namespace tr {
namespace {

constexpr int kThreads = 256;

enum { kModeAuto = 0, kModeTiled = 1, kModeStream = 2 };

__device__ __forceinline__ bool goes_to_stream(int c, int mode) {
  return mode == kModeStream || (mode == kModeAuto && c <= kStreamMaxRows);
}

struct GemmArgs {
  const void* A;        // [R_cap, Kd] rows (Xe for GEMM1, h for GEMM2)
  const void* B;        // [E, Nb, Kd] weights (W1: Nb = 2I, W2: Nb = H)
  void* C;              // [R_cap, Nc] outputs (h: Nc = I, O: Nc = H)
  const int* counts;
  const int* offsets;
  int E;
  int Kd;               // reduction length
  int Nc;               // output columns
  int mode;
};

// Builds in LDS the exclusive prefix of `units(e)` over experts; returns the
// total. `pre` has E+1 entries, `tmp` kThreads/64.
template <typename F>
__device__ int expert_prefix(const int* __restrict__ counts, int E, F units, int* pre, int* tmp) {
  const int per = (E + kThreads - 1) / kThreads;
  int u[4];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = threadIdx.x * per + j;
    u[j] = (j < per && e < E) ? units(counts[e]) : 0;
    sum += u[j];
  }
  int total = 0;
  int off = block_exclusive_scan<kThreads>(sum, tmp, &total);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = threadIdx.x * per + j;
    if (j < per && e < E) {
      pre[e] = off;
      off += u[j];
    }
  }
  if (threadIdx.x == 0) pre[E] = total;
  __syncthreads();
  return total;
}

// Largest e with pre[e] <= v (pre non-decreasing, pre[0] = 0 <= v < pre[E]).
__device__ __forceinline__ int find_expert(const int* pre, int E, int v) {
  int lo = 0, hi = E;  // pre[lo] <= v < pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= v) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// --------------------------------------------------------------------------
// Tiled MFMA kernel (bf16)
// --------------------------------------------------------------------------
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kChunksPerRow = BK / 8;               // 16-byte chunks per tile row
constexpr int kTileChunks = (BM + BN) * kChunksPerRow;  // per stage, 16-byte units
constexpr int kLoadsPerThread = BM * kChunksPerRow / kThreads;  // 8 for A, 8 for B
constexpr int kGroupM = 4;

template <bool kSwiglu>
__global__ __launch_bounds__(kThreads) void gemm_tiled(GemmArgs a, int I) {
  __shared__ u32x4 lds[2][kTileChunks];
  __shared__ int pre[kMaxE + 1];
  __shared__ int tmp[kThreads / kWave];

  const int mode = a.mode;
  const int total_m = expert_prefix(a.counts, a.E, [mode](int c) {
    return (c > 0 && !goes_to_stream(c, mode)) ? (c + BM - 1) / BM : 0;
  }, pre, tmp);
  const int n_cols_per_tile = kSwiglu ? BN / 2 : BN;
  const int NT = (a.Nc + n_cols_per_tile - 1) / n_cols_per_tile;
  const int total = total_m * NT;
  if (total == 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int Kd = a.Kd;
  const int64_t Nb = kSwiglu ? 2 * static_cast<int64_t>(I) : a.Nc;
  const uint16_t* __restrict__ Ab = static_cast<const uint16_t*>(a.A);
  const uint16_t* __restrict__ Bb = static_cast<const uint16_t*>(a.B);
  uint16_t* __restrict__ Cb = static_cast<uint16_t*>(a.C);

  // XCD-aware order: blocks are dealt round-robin to the 8 XCDs; give each
  // XCD a contiguous run of the tile order.
  const int G = gridDim.x;
  int pos = blockIdx.x;
  if ((G & 7) == 0) pos = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  // Per-thread load geometry: chunk column is fixed, rows step by 32.
  const int ld_row = tid >> 3;   // + 32 * j
  const int ld_ch = tid & 7;

  for (int L = pos; L < total; L += G) {
    // tile order: groups of kGroupM m-tiles x all n-tiles, m fastest
    const int group = L / (kGroupM * NT);
    const int first = group * kGroupM;
    const int gsz = min(total_m - first, kGroupM);
    const int within = L - group * kGroupM * NT;
    const int gm = first + within % gsz;
    const int nt = within / gsz;
    const int e = find_expert(pre, a.E, gm);
    const int mt = gm - pre[e];
    const int cnt = a.counts[e];
    const int row0 = a.offsets[e] + mt * BM;
    const int rows_valid = min(BM, cnt - mt * BM);
    const int n0 = nt * n_cols_per_tile;

    // global offsets (elements) of this thread's 8 A rows and 8 B rows
    int64_t aoff[kLoadsPerThread], boff[kLoadsPerThread];
#pragma unroll
    for (int j = 0; j < kLoadsPerThread; ++j) {
      const int r = ld_row + 32 * j;
      const int rr = min(r, rows_valid - 1);
      aoff[j] = static_cast<int64_t>(row0 + rr) * Kd + ld_ch * 8;
      int64_t brow;
      if (kSwiglu) {
        const int half = r >> 7;            // 0: gate rows, 1: up rows
        const int c = min(n0 + (r & 127), I - 1);
        brow = half ? I + c : c;
      } else {
        brow = min(n0 + r, a.Nc - 1);
      }
      boff[j] = (static_cast<int64_t>(e) * Nb + brow) * Kd + ld_ch * 8;
    }

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    u32x4 ra[kLoadsPerThread], rb[kLoadsPerThread];
    auto gload = [&](int k0) {
#pragma unroll
      for (int j = 0; j < kLoadsPerThread; ++j) {
        ra[j] = *reinterpret_cast<const u32x4*>(Ab + aoff[j] + k0);
        rb[j] = *reinterpret_cast<const u32x4*>(Bb + boff[j] + k0);
      }
    };
    auto sstore = [&](int buf) {
#pragma unroll
      for (int j = 0; j < kLoadsPerThread; ++j) {
        const int r = ld_row + 32 * j;
        const int sw = ld_ch ^ (r & 7);
        lds[buf][r * kChunksPerRow + sw] = ra[j];
        lds[buf][(BM + r) * kChunksPerRow + sw] = rb[j];
      }
    };

    const int nk = Kd / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        const int ch = (2 * s + (lane >> 5)) ^ (lane & 7);
        bf16x8 fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = wm * 128 + i * 32 + (lane & 31);
          const u32x4 t = lds[cur][r * kChunksPerRow + ch];
          fa[i] = __builtin_bit_cast(bf16x8, t);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int r;
          if (kSwiglu) r = (j < 2 ? wn * 64 + j * 32 : 128 + wn * 64 + (j - 2) * 32) + (lane & 31);
          else r = wn * 128 + j * 32 + (lane & 31);
          const u32x4 t = lds[cur][(BM + r) * kChunksPerRow + ch];
          fb[j] = __builtin_bit_cast(bf16x8, t);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) sstore(cur ^ 1);
      __syncthreads();
    }

    // epilogue: lane owns column (lane & 31) of each 32x32 block and rows
    // 8*(v/4) + 4*(lane/32) + (v%4)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r >= rows_valid) continue;
        const int64_t orow = static_cast<int64_t>(row0 + r) * a.Nc;
        if (kSwiglu) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + (lane & 31);
            if (col < a.Nc)
              Cb[orow + col] = static_cast<uint16_t>(
                  f32_to_bf16_bits(silu_mul(acc[i][j][v], acc[i][j + 2][v])));
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 128 + j * 32 + (lane & 31);
            if (col < a.Nc) Cb[orow + col] = static_cast<uint16_t>(f32_to_bf16_bits(acc[i][j][v]));
          }
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// Weight-streaming kernel (bf16, experts with few rows)
// --------------------------------------------------------------------------
constexpr int kStreamU = 8;  // k32 blocks per unrolled step

template <bool kSwiglu>
__global__ __launch_bounds__(kThreads) void gemm_stream(GemmArgs a, int I) {
  __shared__ int pre[kMaxE + 1];
  __shared__ int list[kMaxE];
  __shared__ int tmp[kThreads / kWave];
  __shared__ floatx4 red[kThreads / kWave][2][kWave];

  const int mode = a.mode;
  const int n_elig = expert_prefix(a.counts, a.E, [mode](int c) {
    return (c > 0 && goes_to_stream(c, mode)) ? 1 : 0;
  }, pre, tmp);
  if (n_elig == 0) return;
  for (int e = threadIdx.x; e < a.E; e += kThreads)
    if (pre[e + 1] > pre[e]) list[pre[e]] = e;
  __syncthreads();

  const int cols = kSwiglu ? 8 : 16;               // outputs per unit
  const int upe = (a.Nc + cols - 1) / cols;        // units per expert
  const int total = n_elig * upe;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;                         // k group of the lane
  const int arow = lane & 15;                      // operand row of the lane
  const int Kd = a.Kd;
  const int nk32 = Kd / 32;
  const int kb0 = wave * nk32 / 4, kb1 = (wave + 1) * nk32 / 4;
  const int64_t Nb = kSwiglu ? 2 * static_cast<int64_t>(I) : a.Nc;
  const uint16_t* __restrict__ Ab = static_cast<const uint16_t*>(a.A);
  const uint16_t* __restrict__ Bb = static_cast<const uint16_t*>(a.B);
  uint16_t* __restrict__ Cb = static_cast<uint16_t*>(a.C);

  for (int u = blockIdx.x; u < total; u += gridDim.x) {
    const int e = list[u / upe];
    const int c = u % upe;
    const int cnt = a.counts[e];
    const int off = a.offsets[e];
    int64_t wrow;
    if (kSwiglu) {
      const int col = min(c * 8 + (arow & 7), I - 1);
      wrow = arow < 8 ? col : I + col;
    } else {
      wrow = min(c * 16 + arow, a.Nc - 1);
    }
    const uint16_t* wp = Bb + (static_cast<int64_t>(e) * Nb + wrow) * Kd;

    for (int tb = 0; tb < cnt; tb += 32) {
      const uint16_t* xp[2];
      bool xv[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int tok = tb + q * 16 + arow;
        xv[q] = tok < cnt;
        xp[q] = Ab + static_cast<int64_t>(off + (xv[q] ? tok : 0)) * Kd;
      }
      floatx4 acc[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
      int kb = kb0;
      for (; kb + kStreamU <= kb1; kb += kStreamU) {
        // lane group g reads 8*kStreamU contiguous k; step j of the group
        // pairs the j-th 8-element piece of every lane in both operands
        const int k = kb * 32 + g * 8 * kStreamU;
        u32x4 wa[kStreamU], xb[2][kStreamU];
#pragma unroll
        for (int j = 0; j < kStreamU; ++j) wa[j] = *reinterpret_cast<const u32x4*>(wp + k + j * 8);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int j = 0; j < kStreamU; ++j)
            xb[q][j] = xv[q] ? *reinterpret_cast<const u32x4*>(xp[q] + k + j * 8)
                             : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < kStreamU; ++j)
#pragma unroll
          for (int q = 0; q < 2; ++q)
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, wa[j]), __builtin_bit_cast(bf16x8, xb[q][j]), acc[q],
                0, 0, 0);
      }
      for (; kb < kb1; ++kb) {
        const int k = kb * 32 + g * 8;
        const u32x4 wa = *reinterpret_cast<const u32x4*>(wp + k);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const u32x4 xb = xv[q] ? *reinterpret_cast<const u32x4*>(xp[q] + k) : u32x4{0, 0, 0, 0};
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, wa), __builtin_bit_cast(bf16x8, xb), acc[q], 0, 0, 0);
        }
      }
      red[wave][0][lane] = acc[0];
      red[wave][1][lane] = acc[1];
      __syncthreads();
      if (wave == 0) {
        // output element (row 4*g + v, token lane & 15) of each token group
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int tok = tb + q * 16 + (lane & 15);
          floatx4 s = red[0][q][lane];
#pragma unroll
          for (int w = 1; w < kThreads / kWave; ++w) s += red[w][q][lane];
          if (kSwiglu) {
            floatx4 up = red[0][q][lane ^ 32];
#pragma unroll
            for (int w = 1; w < kThreads / kWave; ++w) up += red[w][q][lane ^ 32];
            if (lane < 32 && tok < cnt) {
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const int col = c * 8 + 4 * g + v;
                if (col < I)
                  Cb[static_cast<int64_t>(off + tok) * a.Nc + col] =
                      static_cast<uint16_t>(f32_to_bf16_bits(silu_mul(s[v], up[v])));
              }
            }
          } else if (tok < cnt) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int col = c * 16 + 4 * g + v;
              if (col < a.Nc)
                Cb[static_cast<int64_t>(off + tok) * a.Nc + col] =
                    static_cast<uint16_t>(f32_to_bf16_bits(s[v]));
            }
          }
        }
      }
      __syncthreads();
    }
  }
}

// --------------------------------------------------------------------------
// fp32 kernel: 32 rows x 32 outputs per tile, plain FMAs in k order
// --------------------------------------------------------------------------
constexpr int F_BM = 32, F_BN = 32, F_BK = 32;

template <bool kSwiglu>
__global__ __launch_bounds__(kThreads) void gemm_f32(GemmArgs a, int I) {
  __shared__ int pre[kMaxE + 1];
  __shared__ int tmp[kThreads / kWave];
  __shared__ float As[F_BM][F_BK + 1];
  __shared__ float Bs[2 * F_BN][F_BK + 1];

  const int total_m = expert_prefix(a.counts, a.E, [](int c) {
    return c > 0 ? (c + F_BM - 1) / F_BM : 0;
  }, pre, tmp);
  const int NT = (a.Nc + F_BN - 1) / F_BN;
  const int total = total_m * NT;
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;   // rows 2*ty+{0,1}, cols 2*tx+{0,1}
  const int Kd = a.Kd;
  const int64_t Nb = kSwiglu ? 2 * static_cast<int64_t>(I) : a.Nc;
  const int nbrows = kSwiglu ? 2 * F_BN : F_BN;
  const float* __restrict__ Af = static_cast<const float*>(a.A);
  const float* __restrict__ Bf = static_cast<const float*>(a.B);
  float* __restrict__ Cf = static_cast<float*>(a.C);

  for (int L = blockIdx.x; L < total; L += gridDim.x) {
    const int gm = L / NT, nt = L % NT;
    const int e = find_expert(pre, a.E, gm);
    const int mt = gm - pre[e];
    const int row0 = a.offsets[e] + mt * F_BM;
    const int rows_valid = min(F_BM, a.counts[e] - mt * F_BM);
    const int n0 = nt * F_BN;
    float accg[2][2] = {{0, 0}, {0, 0}}, accu[2][2] = {{0, 0}, {0, 0}};
    for (int k0 = 0; k0 < Kd; k0 += F_BK) {
      for (int i = tid; i < F_BM * F_BK; i += kThreads) {
        const int r = i / F_BK, k = i % F_BK;
        const int rr = min(r, rows_valid - 1);
        As[r][k] = (k0 + k < Kd) ? Af[static_cast<int64_t>(row0 + rr) * Kd + k0 + k] : 0.0f;
      }
      for (int i = tid; i < nbrows * F_BK; i += kThreads) {
        const int r = i / F_BK, k = i % F_BK;
        int64_t brow;
        if (kSwiglu) {
          const int c = min(n0 + (r % F_BN), I - 1);
          brow = r < F_BN ? c : I + c;
        } else {
          brow = min(n0 + r, a.Nc - 1);
        }
        Bs[r][k] = (k0 + k < Kd) ? Bf[(static_cast<int64_t>(e) * Nb + brow) * Kd + k0 + k] : 0.0f;
      }
      __syncthreads();
      for (int k = 0; k < F_BK; ++k) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            accg[i][j] = fmaf(As[2 * ty + i][k], Bs[2 * tx + j][k], accg[i][j]);
            if (kSwiglu) accu[i][j] = fmaf(As[2 * ty + i][k], Bs[F_BN + 2 * tx + j][k], accu[i][j]);
          }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 2 * ty + i, col = n0 + 2 * tx + j;
        if (r < rows_valid && col < a.Nc)
          Cf[static_cast<int64_t>(row0 + r) * a.Nc + col] =
              kSwiglu ? silu_mul(accg[i][j], accu[i][j]) : accg[i][j];
      }
  }
}

}  // namespace

hipError_t grouped_gemm(const tr_moe_plan& p, const void* w1, const void* w2, int parts,
                        hipStream_t st) {
  const tr_moe_desc& d = p.d;
  if (d.T == 0) return hipSuccess;
  const int cus = device_cu_count();
  const int mode = (d.flags & TR_FLAG_GEMM_FORCE_STREAM) ? kModeStream
                   : (d.flags & TR_FLAG_GEMM_FORCE_TILED) ? kModeTiled : kModeAuto;
  const int E = d.E;
  const int I = static_cast<int>(d.I);
  const bool up = parts & kGemmUp, down = parts & kGemmDown;
  GemmArgs g1{p.Xe, w1, p.h, p.counts, p.offsets, E, static_cast<int>(d.H), I, mode};
  GemmArgs g2{p.h, w2, p.O, p.counts, p.offsets, E, I, static_cast<int>(d.H), mode};
  hipError_t err;

  if (d.dtype == TR_F32) {
    const int64_t tiles1 = (cdiv(p.R_cap, F_BM) + E) * cdiv(I, F_BN);
    const int64_t tiles2 = (cdiv(p.R_cap, F_BM) + E) * cdiv(d.H, F_BN);
    const unsigned grid1 = static_cast<unsigned>(tiles1 < cus * 8 ? tiles1 : cus * 8);
    const unsigned grid2 = static_cast<unsigned>(tiles2 < cus * 8 ? tiles2 : cus * 8);
    if (up) {
      hipLaunchKernelGGL(gemm_f32<true>, dim3(grid1), dim3(kThreads), 0, st, g1, I);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (down) {
      hipLaunchKernelGGL(gemm_f32<false>, dim3(grid2), dim3(kThreads), 0, st, g2, I);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
  }

  // tiled: persistent, one block per CU; stream: persistent, 8 blocks per CU
  const int64_t mt_cap = cdiv(p.R_cap, BM) + E;
  const int64_t t1 = mt_cap * cdiv(I, BN / 2), t2 = mt_cap * cdiv(d.H, BN);
  const unsigned gt1 = static_cast<unsigned>(t1 < cus ? t1 : cus);
  const unsigned gt2 = static_cast<unsigned>(t2 < cus ? t2 : cus);
  const int64_t u1 = static_cast<int64_t>(E) * cdiv(I, 8), u2 = static_cast<int64_t>(E) * cdiv(d.H, 16);
  const unsigned gs1 = static_cast<unsigned>(u1 < cus * 8 ? u1 : cus * 8);
  const unsigned gs2 = static_cast<unsigned>(u2 < cus * 8 ? u2 : cus * 8);
  if (up && mode != kModeStream) {
    hipLaunchKernelGGL(gemm_tiled<true>, dim3(gt1), dim3(kThreads), 0, st, g1, I);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (up && mode != kModeTiled) {
    hipLaunchKernelGGL(gemm_stream<true>, dim3(gs1), dim3(kThreads), 0, st, g1, I);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (down && mode != kModeStream) {
    hipLaunchKernelGGL(gemm_tiled<false>, dim3(gt2), dim3(kThreads), 0, st, g2, I);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (down && mode != kModeTiled) {
    hipLaunchKernelGGL(gemm_stream<false>, dim3(gs2), dim3(kThreads), 0, st, g2, I);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace tr
