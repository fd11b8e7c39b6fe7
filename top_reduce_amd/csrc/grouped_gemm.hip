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
  const void* A;        // [a_rows, Kd] rows (Xe for GEMM1, h for GEMM2)
  const void* B;        // [E, Nb, Kd] weights (W1: Nb = 2I, W2: Nb = H)
  void* C;              // [R_cap, Nc] outputs (h: Nc = I, O: Nc = H)
  const int* counts;
  const int* offsets;
  int E;
  int Kd;               // reduction length
  int Nc;               // output columns
  int mode;
  int64_t a_rows;       // rows allocated in A: R_cap + BM
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
static_assert(BM <= kRowPad, "A buffers must carry BM spare rows");
static_assert(BN == kColMultiple, "the H granularity must match the tile");
constexpr int kCpr = BK / 8;                          // 16-byte chunks per tile row (8)
constexpr int kRegion = BM * kCpr;                    // 16-byte units per operand per stage
constexpr int kStageUnits = 2 * kRegion;              // A then B: 64 KiB per stage
constexpr int kWavesT = kThreads / kWave;             // 4
constexpr int kDmaPerWave = kStageUnits / kWave / kWavesT;  // 16 x 1 KiB per wave per stage
constexpr int kSub = BK / 16;                         // MFMA k-steps per stage (4)
[[maybe_unused]] constexpr int kGroupM = 4;
// Word 3 of a raw buffer resource on gfx950 (32-bit data format, no swizzle).
[[maybe_unused]] constexpr int kBufferFlags = 0x00020000;
// s_waitcnt immediates (gfx9 encoding; fields not waited on are at maximum):
// vmcnt(kDmaPerWave) = vmcnt(16), and vmcnt(0) + lgkmcnt(0).
[[maybe_unused]] constexpr int kWaitVm16 = 0x4000 | 0x0F70;
[[maybe_unused]] constexpr int kWaitVm2Lgkm0 = 0x0072;
static_assert(kDmaPerWave == 16, "kWaitVm16 encodes vmcnt(16)");
// L2 prefetch: k-tile kt + 2 + kPrefetchAhead is touched (one dword per
// 128-byte line, all BM + BN rows) when k-tile kt + 2 is requested, so the
// real DMA later finds its lines in L2. Two 64-line DMAs per wave.
constexpr int kPrefetchAhead = 2;
constexpr int kPrefetchPerWave = 2;
static_assert(kPrefetchPerWave == 2, "kWaitVm2Lgkm0 encodes vmcnt(2)");

// Row r of a stage keeps its logical 16-byte chunk c at physical chunk
// c ^ (r & 7): the 8 rows one LDS cycle serves hit 8 distinct bank groups.

// Workgroup barrier that orders LDS accesses for the compiler only. It does
// not wait for in-flight LDS DMA (callers wait with vmcnt first).
[[maybe_unused]] __device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// Two LDS stages as distinct objects: reads of one provably do not alias DMA
// into the other, so the compiler adds no wait for in-flight DMA before them.
__shared__ u32x4 g_stage0[kStageUnits];
__shared__ u32x4 g_stage1[kStageUnits];
// Destination of the L2-prefetch DMAs: written, never read.
__shared__ uint32_t g_prefetch_sink[kWave];

template <int S>
__device__ __forceinline__ u32x4* stage_ptr() { return S == 0 ? g_stage0 : g_stage1; }
[[maybe_unused]] __device__ __forceinline__ u32x4* stage_ptr_rt(int s) {
  return s == 0 ? g_stage0 : g_stage1;
}

// The buffer-resource type exists only in the device compilation pass, so
// the per-tile context and the pipeline helpers are device-pass only.
#if defined(__HIP_DEVICE_COMPILE__)
template <bool kSwiglu>
struct TileCtx {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff;                 // this lane's byte offset for DMA 0 of a stage
  uint32_t dma_stride;           // bytes between the rows of DMA j and j + 1
  uint32_t pf_off;               // this lane's row (prefetch DMA 0), bytes
  uint32_t pf_stride;            // bytes between the rows of prefetch DMA 0 and 1
  int dma_dst;
  int a_frag, b_frag;
  int frag_ch[kSub];
  bf16x8 fa[2][4], fb[2][4];     // fragments of two MFMA k-steps
  floatx16 acc[4][4];
};

// Stage S <- k-tile kt: 16 DMA of 1 KiB (8 rows x 128 B) per wave.
template <int S, bool kSwiglu>
__device__ __forceinline__ void issue_stage(TileCtx<kSwiglu>& c, int kt) {
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        c.rsrc, (lds_void*)(stage_ptr<S>() + c.dma_dst + j * 8 * kCpr), 16, c.voff,
        kt * BK * 2 + j * c.dma_stride, 0, 0);
}

// Pull the lines of k-tile kt into L2: lane -> one row, one dword per line.
template <bool kSwiglu>
__device__ __forceinline__ void prefetch_l2(TileCtx<kSwiglu>& c, int kt) {
#pragma unroll
  for (int q = 0; q < kPrefetchPerWave; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsrc, (lds_void*)g_prefetch_sink, 4, c.pf_off,
                                             kt * BK * 2 + q * c.pf_stride, 0, 0);
}

// Fragments of MFMA k-step `sub` of stage S into register set P.
template <int S, int P, bool kSwiglu>
__device__ __forceinline__ void read_frags(TileCtx<kSwiglu>& c, int sub) {
  const u32x4* base = stage_ptr<S>();
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c.fa[P][i] = __builtin_bit_cast(bf16x8, base[c.a_frag + i * 32 * kCpr + c.frag_ch[sub]]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rb = kSwiglu ? (j < 2 ? j * 32 : 128 + (j - 2) * 32) : j * 32;
    c.fb[P][j] = __builtin_bit_cast(bf16x8, base[c.b_frag + rb * kCpr + c.frag_ch[sub]]);
  }
}

template <int P, bool kSwiglu>
__device__ __forceinline__ void mma(TileCtx<kSwiglu>& c) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c.fa[P][i], c.fb[P][j], c.acc[i][j], 0, 0, 0);
}

// One k-tile held in stage S, with its first k-step's fragments already in
// register set 0. The DMA of the next k-tile into the other stage is in
// flight. Fragment reads run one MFMA k-step ahead; before the last k-step's
// MFMAs the wave waits for the next k-tile's DMA and drains its LDS reads,
// all waves meet, the next k-tile's first fragments are read and stage S is
// refilled with k-tile kt + 2, so the barrier hides behind 16 MFMAs.
// The scheduling barriers pin this order: the compiler would otherwise sink
// each fragment read next to its first use and wait on it, exposing LDS
// latency every few MFMAs.
template <int S, bool kSwiglu>
__device__ __forceinline__ void ring_step(TileCtx<kSwiglu>& c, int kt, int nk) {
  read_frags<S, 1>(c, 1);
  __builtin_amdgcn_sched_barrier(0);
  mma<0>(c);
  __builtin_amdgcn_sched_barrier(0);
  read_frags<S, 0>(c, 2);
  __builtin_amdgcn_sched_barrier(0);
  mma<1>(c);
  __builtin_amdgcn_sched_barrier(0);
  read_frags<S, 1>(c, 3);
  __builtin_amdgcn_sched_barrier(0);
  mma<0>(c);
  __builtin_amdgcn_sched_barrier(0);
  // k-tile kt+1 landed (only its prefetch may still be in flight); stage S
  // fully read by this wave
  __builtin_amdgcn_s_waitcnt(kWaitVm2Lgkm0);
  lds_barrier();
  read_frags<1 - S, 0>(c, 0);
  issue_stage<S>(c, min(kt + 2, nk - 1));
  prefetch_l2(c, min(kt + 2 + kPrefetchAhead, nk - 1));
  __builtin_amdgcn_sched_barrier(0);
  mma<1>(c);
  __builtin_amdgcn_sched_barrier(0);
}
#endif  // __HIP_DEVICE_COMPILE__

template <bool kSwiglu>
__global__ __launch_bounds__(kThreads) void gemm_tiled(GemmArgs a, int I) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ int pre[kMaxE + 1];
  __shared__ int tmp[kWavesT];

  const int mode = a.mode;
  const int total_m = expert_prefix(a.counts, a.E, [mode](int c) {
    return (c > 0 && !goes_to_stream(c, mode)) ? (c + BM - 1) / BM : 0;
  }, pre, tmp);
  constexpr int kOutCols = kSwiglu ? BN / 2 : BN;   // output columns per tile
  const int NT = (a.Nc + kOutCols - 1) / kOutCols;
  const int total = total_m * NT;
  if (total == 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  for (int L = pos; L < total; L += G) {
    // Lane geometry is recomputed per tile from an opaque copy of the lane id,
    // so its registers are not held across the epilogue.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    TileCtx<kSwiglu> c;
    // DMA geometry: waves 0-1 fill the A region, waves 2-3 the B region. DMA j
    // of a wave writes 1 KiB = 8 rows x 8 chunks: lane -> (row lane / 8,
    // physical chunk lane % 8), so the lane fetches logical chunk
    // (lane % 8) ^ (row % 8) = (lane % 8) ^ (lane / 8).
    const int dma_b = wave >> 1;
    const int dma_row0 = (wave & 1) * (BM / 2) + (ln >> 3);     // + 8 j
    const int dma_chunk = (ln & 7) ^ (ln >> 3);
    c.dma_dst = dma_b * kRegion + (wave & 1) * (BM / 2) * kCpr;
    // Fragments: lane reads row (lane & 31) of a 32-row block at logical
    // chunk 2 s + lane / 32 in MFMA k-step s.
#pragma unroll
    for (int s = 0; s < kSub; ++s)
      c.frag_ch[s] = (ln & 31) * kCpr + ((2 * s + (ln >> 5)) ^ (ln & 7));
    c.a_frag = wm * 128 * kCpr;
    c.b_frag = kRegion + (kSwiglu ? wn * 64 : wn * 128) * kCpr;

    // tile order: groups of kGroupM m-tiles x all n-tiles, m fastest
    const int group = L / (kGroupM * NT);
    const int first = group * kGroupM;
    const int gsz = min(total_m - first, kGroupM);
    const int within = L - group * kGroupM * NT;
    const int gm = first + within % gsz;
    const int nt = within / gsz;
    // tile parameters are block-uniform; say so, so that the buffer
    // resources below live in scalar registers
    const int e = __builtin_amdgcn_readfirstlane(find_expert(pre, a.E, gm));
    const int mt = __builtin_amdgcn_readfirstlane(gm - pre[e]);
    const int cnt = __builtin_amdgcn_readfirstlane(a.counts[e]);
    const int row0 = __builtin_amdgcn_readfirstlane(a.offsets[e]) + mt * BM;
    const int rows_valid = min(BM, cnt - mt * BM);
    const int n0 = nt * kOutCols;

    // Buffer resources over this tile's A rows and expert e's weights. Every
    // DMA address is in bounds by construction: the A buffers (Xe, h) carry
    // BM spare rows past R_cap, so a tile may read BM rows from any segment
    // start (rows past the segment only feed discarded outputs), and the
    // weight rows of a tile never pass the expert's 2I (or H) rows because I
    // is a multiple of BN / 2 and H of BN. Row offsets go in the scalar
    // offset, so a lane keeps a single offset register.
    const uint64_t a_left = (static_cast<uint64_t>(a.a_rows) - row0) * Kd * 2;
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(Ab + static_cast<int64_t>(row0) * Kd), 0,
        static_cast<int>(a_left < 0xffffffffull ? a_left : 0xffffffffull), kBufferFlags);
    const uint64_t b_size = static_cast<uint64_t>(Nb) * Kd * 2;
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(Bb + static_cast<int64_t>(e) * Nb * Kd), 0,
        static_cast<int>(b_size < 0xffffffffull ? b_size : 0xffffffffull), kBufferFlags);
    c.rsrc = dma_b ? rB : rA;
    int row = dma_row0;                          // A: tile row of DMA 0
    if (dma_b) {
      if (kSwiglu) row = (wave & 1) ? I + n0 + (ln >> 3) : n0 + (ln >> 3);   // gate | up
      else row = n0 + dma_row0;
    }
    c.voff = (static_cast<uint32_t>(row) * Kd + dma_chunk * 8) * 2;
    c.dma_stride = 8u * Kd * 2;
    // prefetch rows: this wave's 128 rows of its operand, 64 per DMA
    int pf_row = (wave & 1) * (BM / 2) + ln;                       // A tile row
    if (dma_b) {
      if (kSwiglu) pf_row = (wave & 1) ? I + n0 + ln : n0 + ln;   // gate | up
      else pf_row = n0 + pf_row;
    }
    c.pf_off = static_cast<uint32_t>(pf_row) * Kd * 2;
    c.pf_stride = static_cast<uint32_t>(kWave) * Kd * 2;
    // Accumulators start at zero through an MFMA with zero operands: the
    // result lands in accumulation registers directly, instead of 256 zeros
    // built in ordinary vector registers first.
    {
      bf16x8 zf;
      int zero = 0;
      asm volatile("" : "+v"(zero));
#pragma unroll
      for (int q = 0; q < 8; ++q) zf[q] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(zero));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          c.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zf, zf, floatx16{}, 0, 0, 0);
    }

    // Two LDS stages: k-tile kt+1 streams in while k-tile kt is multiplied.
    // Tiles past the end re-read the last one (uniform control flow); their
    // data is never used.
    const int nk = Kd / BK;
    issue_stage<0>(c, 0);
    issue_stage<1>(c, min(1, nk - 1));
    __builtin_amdgcn_s_waitcnt(kWaitVm16);      // k-tile 0 (own DMA)
    prefetch_l2(c, min(2, nk - 1));
    prefetch_l2(c, min(3, nk - 1));
    lds_barrier();
    read_frags<0, 0>(c, 0);
    for (int kt = 0; kt < nk; kt += 2) {
      ring_step<0>(c, kt, nk);
      if (kt + 1 < nk) ring_step<1>(c, kt + 1, nk);
    }
    __builtin_amdgcn_s_waitcnt(0);              // drain the ring before reuse
    __syncthreads();

    // Epilogue: stage the bf16 tile in LDS row-major [BM][kOutCols] (rows
    // split evenly over the two stage buffers), then write whole 16-byte
    // chunks of rows. Lane owns column (lane & 31) of each 32x32 block and
    // rows 8 (v / 4) + 4 (lane / 32) + (v % 4).
    constexpr int kRowsPerStage = kStageUnits * 8 / kOutCols;   // 128 or 256
    constexpr int kBlocksPerStage = kRowsPerStage / 32;          // 32-row blocks
    // This wave's rows wm*128 + [0, 128) sit in buffer wm*128 / kRowsPerStage.
    const int lane_off = 4 * (ln >> 5) * kOutCols + (kSwiglu ? wn * 64 : wn * 128) + (ln & 31);
    uint16_t* ob = reinterpret_cast<uint16_t*>(stage_ptr_rt((wm * 128) / kRowsPerStage)) +
                   ((wm * 128) % kRowsPerStage) * kOutCols + lane_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t* base = ob + i * 32 * kOutCols;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        uint16_t* orow = base + (8 * (v >> 2) + (v & 3)) * kOutCols;
        if (kSwiglu) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
            orow[j * 32] = static_cast<uint16_t>(
                f32_to_bf16_bits(silu_mul(c.acc[i][j][v], c.acc[i][j + 2][v])));
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            orow[j * 32] = static_cast<uint16_t>(f32_to_bf16_bits(c.acc[i][j][v]));
        }
        // convert a few accumulators at a time: bounded register pressure
        if ((v & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
    (void)kBlocksPerStage;
    __syncthreads();
    constexpr int kOutChunks = kOutCols / 8;   // 16-byte chunks per output row
    for (int q = tid; q < BM * kOutChunks; q += kThreads) {
      const int r = q / kOutChunks, ch = q % kOutChunks, col = n0 + ch * 8;
      if (r < rows_valid && col < a.Nc)
        *reinterpret_cast<u32x4*>(Cb + static_cast<int64_t>(row0 + r) * a.Nc + col) =
            stage_ptr_rt(r / kRowsPerStage)[(r % kRowsPerStage) * kOutChunks + ch];
    }
    __syncthreads();
  }
#endif  // __HIP_DEVICE_COMPILE__
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
  const int64_t a_rows = p.R_cap + kRowPad;
  GemmArgs g1{p.Xe, w1, p.h, p.counts, p.offsets, E, static_cast<int>(d.H), I, mode, a_rows};
  GemmArgs g2{p.h, w2, p.O, p.counts, p.offsets, E, I, static_cast<int>(d.H), mode, a_rows};
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
