// moe_grouped_gemm: the local experts' SwiGLU MLP over the expert-contiguous
// rows Xe, or over x read through the route table (DeepEP issue #48 answer: a
// grouped GEMM over expanded tokens).
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
//    operands staged through two XOR-swizzled LDS stages: activation rows by
//    buffer->LDS DMA one k-tile ahead, weight rows through registers loaded
//    two k-tiles ahead and written to LDS one k-tile ahead, both spread over
//    the k-steps' MFMAs. With GEMM1 gathering, the activation rows come
//    straight from x through the route table. Tiles are numbered expert-major
//    with groups of 4 m-tiles and handed to the 8 XCDs in contiguous chunks so
//    that concurrent tiles of an XCD share A and B tiles in its L2. For GEMM1
//    each B tile holds 128 gate rows and the matching 128 up rows, so a lane
//    owns gate and up of the same outputs and SwiGLU runs in the epilogue.
//  - gemm_stream: experts with few rows (decode). Weight rows are streamed
//    once from HBM straight into the A operand of v_mfma_f32_16x16x32_bf16;
//    up to 32 token rows ride in the B operand; the reduction dimension is
//    split over the four waves of a block and summed in LDS in a fixed order.
//
// An fp32 variant (gemm_f32) covers fp32 inputs on fp32 MFMA
// (v_mfma_f32_16x16x4_f32), one wave per 16 x 16 output tile.
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
  int64_t a_rows;       // rows allocated in A: R_cap + BM (gather: the rows of x)
  const int* gather;    // GEMM1 straight from the received rows: A row r of the
                        // expanded order is row gather[r] of A (x); NULL: A is Xe
  // GEMM2 with the reduce folded in for received rows with one local slot
  // (rows of tiled experts only): row r goes to y[dst[r] / K] weighted by
  // wts[dst[r]] (dst[r] >= 0), not O
  const int* dst;       // the plan's row_dst, or NULL: every row goes to O
  const float* wts;     // [T, K] gate weights, or NULL for weight 1
  void* y;              // [T, Nc]
  int K;
  int64_t T;
  // the number of experts this launch's kernel takes, counted by the route
  // scan (plan stats 6: streaming, 7: tiled); a launch with none exits after
  // its first loads. Read by gemm_tiled, gemm_hybrid and gemm_stream (never
  // NULL for them).
  const int* n_take;
};

// Builds in LDS the exclusive prefix of `units(e)` over experts; returns the
// total. `pre` has E+1 entries, `tmp` kBlock/64; E <= 4 kBlock.
template <int kBlock = kThreads, typename F>
__device__ int expert_prefix(const int* __restrict__ counts, int E, F units, int* pre, int* tmp) {
  static_assert(4 * kBlock >= kMaxE, "four experts per thread");
  const int per = (E + kBlock - 1) / kBlock;
  // the counts, loaded unconditionally (index clamped; E >= 1) so that all
  // go out before the first wait, then masked
  int cv[4], u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    cv[j] = j < per ? counts[min(static_cast<int>(threadIdx.x) * per + j, E - 1)] : 0;
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = threadIdx.x * per + j;
    u[j] = (j < per && e < E) ? units(cv[j]) : 0;
    sum += u[j];
  }
  int total = 0;
  int off = block_exclusive_scan<kBlock>(sum, tmp, &total);
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

// silu(g) * u = g u / (1 + e^-g), with the hardware exponential and
// reciprocal (about 1 ulp each, far below the bf16 rounding of the result).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Two floats rounded to bf16 (nearest even) by one hardware conversion; lo in
// bits 0..15.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// --------------------------------------------------------------------------
// Tiled MFMA kernel (bf16)
// --------------------------------------------------------------------------
constexpr int BM = 256, BN = 256, BK = 64;
static_assert(BM <= kRowPad, "A buffers must carry BM spare rows");
static_assert(BN == kColMultiple, "the H granularity must match the tile");
constexpr int kCpr = BK / 8;                          // 16-byte chunks per tile row (8)
constexpr int kRegion = BM * kCpr;                    // 16-byte units per operand per stage
constexpr int kWavesT = kThreads / kWave;             // 4
constexpr int kGroupM = 4;
// Word 3 of a raw buffer resource on gfx950 (32-bit data format, no swizzle).
constexpr int kBufferFlags = 0x00020000;

// s_waitcnt immediate (gfx9 encoding) for vmcnt(n) with lgkmcnt(0) or with
// no lgkm wait; expcnt is never waited on.
__host__ __device__ constexpr int waitcnt_vm(int n, bool lgkm0) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | ((lgkm0 ? 0 : 15) << 8);
}

// Row r of a stage keeps its logical 16-byte chunk c at physical chunk
// c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1). gfx950's LDS has 64 banks: a
// 16-byte fragment read serves 16 lanes (16 rows) per cycle, rows r and r + 1
// land in opposite bank halves, and f is distinct over the 8 even rows and
// over the 8 odd rows of any 16, so the reads are conflict-free.

// Workgroup barrier that orders LDS accesses for the compiler only. It does
// not wait for in-flight LDS DMA (callers wait with vmcnt first).
[[maybe_unused]] __device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// Two LDS stages, each an activation half and a weight half, all distinct
// objects: an access to one provably does not alias DMA into another, so the
// compiler adds no wait for in-flight DMA before it.
__shared__ u32x4 g_a0[kRegion], g_b0[kRegion];
__shared__ u32x4 g_a1[kRegion], g_b1[kRegion];

template <int S>
__device__ __forceinline__ u32x4* stage_a() { return S == 0 ? g_a0 : g_a1; }
template <int S>
__device__ __forceinline__ u32x4* stage_b() { return S == 0 ? g_b0 : g_b1; }

// The buffer-resource type exists only in the device compilation pass, so
// the tile state and the pipeline helpers are device-pass only.
#if defined(__HIP_DEVICE_COMPILE__)

// Operand staging. Each wave moves 8 pieces (1 KiB = 8 rows x 128 B each) of
// the activation tile and 8 of the weight tile per k-tile. The activation
// pieces go straight to LDS by buffer->LDS DMA, issued once the stage is free
// (one k-step to land). The weight pieces go through registers: loaded four
// k-tiles ahead, written to LDS two k-steps later (two k-steps to land).
// Weight rows are the larger share of the L2 misses. The limit here is the
// number of requests a CU keeps in flight times their L2 latency, so deeper
// staging (both operands through registers) measured no faster.
constexpr int kPieces = 8;

// Where one tile's operands come from, for this wave and lane. Pieces are 8
// rows apart. Weight pieces: a lane keeps one byte offset for even and one
// for odd pieces (the swizzle differs) and the pieces' row offsets go in the
// scalar offset. Activation pieces: a lane keeps one offset per piece, so that
// a row past the segment can be given an offset past the buffer (the range
// check covers the vector offset only), whose DMA writes zeros; gathered rows
// are arbitrary anyway.
template <bool kGather>
struct TileSrc {
  __amdgpu_buffer_rsrc_t d_rsrc, r_rsrc;   // activations (DMA), weights (registers)
  uint32_t d_voff[kPieces];  // this lane's activation offsets, k-tile 0
  uint32_t r_voff, r_voff1; // this lane's byte offset in weight piece 0 / 1, k-tile 0
  uint32_t stride;          // bytes between pieces j and j + 1 (8 rows)
  __device__ __forceinline__ uint32_t a_voff(int j) const { return d_voff[j]; }
  __device__ __forceinline__ uint32_t a_soff(int) const { return 0u; }
};

struct TileInfo {
  int e, row0, rows_valid, n0;
};

// Lane geometry, fixed for the whole kernel.
struct Geo {
  int d_dst;            // 16-byte unit of this wave's DMA piece 0 (DMA base)
  int r_dst;            // 16-byte unit of this lane's part of register piece 0
  int a_frag, b_frag;   // 16-byte unit of this wave's first A / B fragment row
  int frag_ch[BK / 16]; // per MFMA k-step: row-in-block * 8 + swizzled chunk
};

struct Frags {
  bf16x8 fa[2][4], fb[2][4];   // fragments of two MFMA k-steps
  floatx16 acc[4][4];          // acc[i][j]: weight block j x row block i
};

// One wave's weight pieces of a k-tile, in registers.
struct Regs {
  u32x4 v[kPieces];
};

// Fragments of MFMA k-step `sub` of stage S into register set P.
template <int S, int P, bool kSwiglu>
__device__ __forceinline__ void read_frags(Frags& f, const Geo& g, int sub) {
  const u32x4* sa = stage_a<S>();
  const u32x4* sb = stage_b<S>();
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.fa[P][i] = __builtin_bit_cast(bf16x8, sa[g.a_frag + i * 32 * kCpr + g.frag_ch[sub]]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rb = kSwiglu ? (j < 2 ? j * 32 : 128 + (j - 2) * 32) : j * 32;
    f.fb[P][j] = __builtin_bit_cast(bf16x8, sb[g.b_frag + rb * kCpr + g.frag_ch[sub]]);
  }
}

// The weight fragment is the MFMA's A operand: a lane then holds four
// consecutive output columns of one row, ready for wide stores.
template <int P>
__device__ __forceinline__ void mma(Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      f.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.fb[P][j], f.fa[P][i], f.acc[i][j], 0, 0, 0);
}

template <int S, bool G>
__device__ __forceinline__ void dma_a(const Geo& g, const TileSrc<G>& s, int kt, int j) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      s.d_rsrc, (lds_void*)(stage_a<S>() + g.d_dst + j * 8 * kCpr), 16, s.a_voff(j),
      kt * BK * 2 + s.a_soff(j), 0, 0);
}

template <bool G>
__device__ __forceinline__ u32x4 load_b(const TileSrc<G>& s, int kt, int j) {
  return __builtin_amdgcn_raw_buffer_load_b128(s.r_rsrc, (j & 1) ? s.r_voff1 : s.r_voff, kt * BK * 2 + j * s.stride, 0);
}

template <int S>
__device__ __forceinline__ void write_b(const Geo& g, const u32x4& v, int j) {
  stage_b<S>()[g.r_dst + j * 8 * kCpr] = v;
}

// The 16 MFMAs of register set P with the 8 activation DMAs of k-tile `dkt`
// of `ds` into stage S between them.
template <int P, int S, bool G>
__device__ __forceinline__ void mma_dma(Frags& f, const Geo& g, const TileSrc<G>& ds, int dkt) {
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int i = m >> 2, j = m & 3;
    f.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.fb[P][j], f.fa[P][i], f.acc[i][j], 0, 0, 0);
    if ((m & 1) == 0) dma_a<S>(g, ds, dkt, m >> 1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The 16 MFMAs of register set P with weight pieces [J0, J0 + N) (N <= 3)
// spread between them: each piece held in `r` goes to stage T, then its
// register is reloaded with the piece of k-tile `lkt` of `ls` (the compiler's
// per-register waits gate each LDS write on its own load only).
template <int P, int T, int J0, int N, bool G>
__device__ __forceinline__ void mma_wl(Frags& f, Regs& r, const Geo& g, const TileSrc<G>& ls,
                                       int lkt) {
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int i = m >> 2, j = m & 3;
    f.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.fb[P][j], f.fa[P][i], f.acc[i][j], 0, 0, 0);
    if (m % 5 == 1 && m / 5 < N) {
      write_b<T>(g, r.v[J0 + m / 5], J0 + m / 5);
      r.v[J0 + m / 5] = load_b(ls, lkt, J0 + m / 5);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Step kt of the ring: k-tile kt in stage S (S = kt % 2), its first k-step's
// fragments already in register set 0; the activations of k-tile kt + 1 in
// flight into stage 1 - S and its weights in `r`. Fragment reads run one
// MFMA k-step ahead (the scheduling barriers keep the compiler from sinking
// each read next to its use).
//  - The first three k-steps' MFMAs carry the weights of k-tile kt + 1 from
//    `r` into stage 1 - S (no wave reads it during this step) and the loads
//    of k-tile kt + 3 (`lkt` of `ls`) into the freed registers.
//  - Then the wave waits for its activation DMA of k-tile kt + 1 (the weight
//    loads issued after it, and the previous tile's kStores output stores if
//    `after_stores`, may stay in flight), drains its LDS traffic, meets the
//    other waves and reads the next k-tile's first fragments.
//  - The last k-step's MFMAs carry the activation DMA of k-tile kt + 2
//    (`dkt` of `ds`) into stage S, which every wave has now finished reading.
//
// The CU's vector memory path moves about 64 bytes a clock, so a k-tile's
// 64 KiB of operand traffic takes about as long as a k-step's MFMAs, and LDS
// writes compete with the fragment reads: issued together in one k-step they
// stall the MFMAs queued behind them; spread over the k-tile they overlap.
template <int S, bool kSwiglu, int kStores, bool G>
__device__ __forceinline__ void ring_step(Frags& f, const Geo& g, Regs& r, bool after_stores,
                                          const TileSrc<G>& ds, int dkt, const TileSrc<G>& ls,
                                          int lkt) {
  read_frags<S, 1, kSwiglu>(f, g, 1);
  __builtin_amdgcn_sched_barrier(0);
  mma_wl<0, 1 - S, 0, 3>(f, r, g, ls, lkt);
  __builtin_amdgcn_sched_barrier(0);
  read_frags<S, 0, kSwiglu>(f, g, 2);
  __builtin_amdgcn_sched_barrier(0);
  mma_wl<1, 1 - S, 3, 3>(f, r, g, ls, lkt);
  __builtin_amdgcn_sched_barrier(0);
  read_frags<S, 1, kSwiglu>(f, g, 3);
  __builtin_amdgcn_sched_barrier(0);
  mma_wl<0, 1 - S, 6, 2>(f, r, g, ls, lkt);
  __builtin_amdgcn_sched_barrier(0);
  if (after_stores) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kPieces + kStores, true));
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm(kPieces, true));
  lds_barrier();
  read_frags<1 - S, 0, kSwiglu>(f, g, 0);
  __builtin_amdgcn_sched_barrier(0);
  mma_dma<1, S>(f, g, ds, dkt);
  __builtin_amdgcn_sched_barrier(0);
}

// Tile L of the order: groups of kGroupM m-tiles x all n-tiles, m fastest.
// cnt_s / off_s: the experts' counts and segment offsets, copied to LDS so
// that per-tile lookups are LDS reads, not vector loads (whose waits would
// also wait for the loads in flight).
template <int kOutCols>
__device__ __forceinline__ TileInfo tile_info(const GemmArgs& a, const int* pre, const int* cnt_s,
                                              const int* off_s, int total_m, int NT, int L) {
  const int group = L / (kGroupM * NT);
  const int first = group * kGroupM;
  const int gsz = min(total_m - first, kGroupM);
  const int within = L - group * kGroupM * NT;
  const int gm = first + within % gsz;
  const int nt = within / gsz;
  TileInfo t;
  // block-uniform; say so, so that buffer resources live in scalar registers
  t.e = __builtin_amdgcn_readfirstlane(find_expert(pre, a.E, gm));
  const int mt = __builtin_amdgcn_readfirstlane(gm - pre[t.e]);
  const int cnt = __builtin_amdgcn_readfirstlane(cnt_s[t.e]);
  t.row0 = __builtin_amdgcn_readfirstlane(off_s[t.e]) + mt * BM;
  t.rows_valid = min(BM, cnt - mt * BM);
  t.n0 = nt * kOutCols;
  return t;
}

// Operand sources of a tile for this wave. Every address is in bounds by
// construction: the A buffers (Xe, h) carry BM spare rows past R_cap, so a
// tile may read BM rows from any segment start (rows past the segment only
// feed discarded outputs); a gathered A gives those rows an offset past the
// buffer, which the range check turns into zeros without an access; and
// a tile's weight rows never pass the expert's 2I (or H) rows because I is a
// multiple of BN / 2 and H of BN.
template <bool kSwiglu, bool kGather>
__device__ __forceinline__ TileSrc<kGather> tile_src(const GemmArgs& a, const TileInfo& t, int I,
                                                     int wave, int ln) {
  const int Kd = a.Kd;
  const int64_t Nb = kSwiglu ? 2 * static_cast<int64_t>(I) : a.Nc;
  TileSrc<kGather> s;
  const uint16_t* abase = static_cast<const uint16_t*>(a.A);
  uint64_t left = static_cast<uint64_t>(a.a_rows) * Kd * 2;
  if (!kGather) {
    // the tile's rows only: at most BM * Kd * 2 <= 2^31 bytes, so an offset
    // of 2^31 is past the buffer
    abase += static_cast<int64_t>(t.row0) * Kd;
    left -= static_cast<uint64_t>(t.row0) * Kd * 2;
    const uint64_t tile_bytes = static_cast<uint64_t>(BM) * Kd * 2;
    left = left < tile_bytes ? left : tile_bytes;
  }
  s.d_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(abase), 0,
                                               static_cast<int>(left < 0xffffffffull ? left : 0xffffffffull),
                                               kBufferFlags);
  const uint64_t size = static_cast<uint64_t>(Nb) * Kd * 2;
  s.r_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(static_cast<const uint16_t*>(a.B) + static_cast<int64_t>(t.e) * Nb * Kd),
      0, static_cast<int>(size < 0xffffffffull ? size : 0xffffffffull), kBufferFlags);
  // Piece j holds 8 rows x 8 chunks: lane -> (row lane / 8, physical chunk
  // lane % 8), fetching logical chunk (lane % 8) ^ f(row) with f(row) =
  // (lane / 8) ^ (j & 1). This wave's activation rows are wave * 64 + j * 8 +
  // lane / 8 of the tile; its weight rows 64 rows of the B tile.
  const int chunk = (ln & 7) ^ (ln >> 3);
  if (kGather) {
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int lr = wave * 64 + j * 8 + (ln >> 3);
      // a row past the segment gets an offset past the buffer (x is under
      // 2 GiB): its DMA writes zeros, so the MFMAs on it toggle no data bits
      s.d_voff[j] = lr < t.rows_valid
                        ? (static_cast<uint32_t>(a.gather[t.row0 + lr]) * Kd + (chunk ^ (j & 1)) * 8) * 2
                        : 0x80000000u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int lr = wave * 64 + j * 8 + (ln >> 3);
      s.d_voff[j] = lr < t.rows_valid
                        ? (static_cast<uint32_t>(lr) * Kd + (chunk ^ (j & 1)) * 8) * 2
                        : 0x80000000u;
    }
  }
  int b_row;
  if (kSwiglu) b_row = wave < 2 ? t.n0 + wave * 64 : I + t.n0 + (wave - 2) * 64;  // gate | up
  else b_row = t.n0 + wave * 64;
  s.r_voff = (static_cast<uint32_t>(b_row + (ln >> 3)) * Kd + chunk * 8) * 2;
  s.r_voff1 = (static_cast<uint32_t>(b_row + (ln >> 3)) * Kd + (chunk ^ 1) * 8) * 2;
  s.stride = 8u * Kd * 2;
  return s;
}

#endif  // __HIP_DEVICE_COMPILE__

#if defined(__HIP_DEVICE_COMPILE__)
// The experts' counts and segment offsets copied to LDS, and the prefix of
// their m-tiles (experts of the tiled kernel only); returns the m-tiles, or
// -1 without touching LDS when the route scan counted no expert for the
// launch (a.n_take).
__device__ __forceinline__ int gemm_prologue(const GemmArgs& a, int* pre, int* tmp, int* cnt_s,
                                             int* off_s) {
  const int take = *a.n_take;
  // loaded unconditionally (index clamped), and stored to LDS only after
  // the prefix has issued its own loads: one wait for memory in all
  int cv[kMaxE / kThreads], ov[kMaxE / kThreads];
#pragma unroll
  for (int j = 0; j < kMaxE / kThreads; ++j) {
    const int e = min(static_cast<int>(threadIdx.x) + j * kThreads, a.E - 1);
    cv[j] = j * kThreads < a.E ? a.counts[e] : 0;
    ov[j] = j * kThreads < a.E ? a.offsets[e] : 0;
  }
  asm volatile("" : : : "memory");   // the loads above go out before the exit test
  if (take == 0) return -1;
  const int mode = a.mode;
  const int total_m = expert_prefix(a.counts, a.E, [mode](int c) {
    return (c > 0 && !goes_to_stream(c, mode)) ? (c + BM - 1) / BM : 0;
  }, pre, tmp);
#pragma unroll
  for (int j = 0; j < kMaxE / kThreads; ++j) {
    const int e = threadIdx.x + j * kThreads;
    if (e < a.E) {
      cnt_s[e] = cv[j];
      off_s[e] = ov[j];
    }
  }
  __syncthreads();
  return total_m;
}

// GEMM1 and GEMM2 of one forward in three launches, so that the blocks idle
// in GEMM1's last, partly filled round compute GEMM2 tiles instead (a launch
// boundary makes GEMM1's output visible to every XCD):
//   1. GEMM1 tiles [0, R1), R1 the whole rounds on G blocks;
//   2. GEMM1 tiles [R1, total1) on the first total1 - R1 blocks, and on the
//      others GEMM2 tiles [0, n2) of m-tiles whose GEMM1 tiles all lie in
//      [0, R1) (whole groups of kGroupM m-tiles), about as many per block as
//      fit in one GEMM1 tile's time (the ratio of the reduction lengths);
//   3. GEMM2 tiles [n2, total2).
// n2 as a function of the m-tiles, the tiles per m-tile of each GEMM, that
// ratio and G; launches 2 and 3 compute it alike.
__device__ __forceinline__ int early_down_tiles(int total_m, int NT1, int NT2, int ratio, int G) {
  const int total1 = total_m * NT1;
  const int R1 = total1 / G * G;
  const int tail = total1 - R1;
  if (tail == 0 || R1 == 0 || ratio == 0) return 0;
  const int m_done = min(R1 / (kGroupM * NT1) * kGroupM, total_m);
  return min((G - tail) * ratio, m_done * NT2);
}

// The tile loop of gemm_tiles (below). pre / cnt_s / off_s: the LDS tables
// of gemm_prologue. kFused (GEMM2 only): the reduce folded into the epilogue
// for the rows the plan's row_dst names (a.dst non-NULL).
template <bool kSwiglu, bool kGather, bool kFused>
__device__ __forceinline__ void gemm_tiles_impl(const GemmArgs& a, int I, const int* pre,
                                                const int* cnt_s, const int* off_s, int total_m,
                                                int begin, int end, int slot, int nslots) {
  constexpr int kOutCols = kSwiglu ? BN / 2 : BN;   // output columns per tile
  const int NT = (a.Nc + kOutCols - 1) / kOutCols;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nk = a.Kd / BK;                 // even and >= 2: H % 256 == 0, I % 128 == 0
  uint16_t* __restrict__ Cb = static_cast<uint16_t*>(a.C);

  // XCD-aware order: blocks are dealt round-robin to the 8 XCDs; give each
  // XCD a contiguous run of the tile order.
  const int G = nslots;
  int pos = slot;
  if ((G & 7) == 0) pos = (slot & 7) * (G >> 3) + (slot >> 3);
  if (pos >= end - begin) return;
  pos += begin;
  const int total = end;

  Geo g;
  g.d_dst = wave * 64 * kCpr;
  g.r_dst = wave * 64 * kCpr + lane;
#pragma unroll
  for (int s = 0; s < BK / 16; ++s)
    g.frag_ch[s] = (lane & 31) * kCpr + ((2 * s + (lane >> 5)) ^ ((lane & 7) ^ ((lane >> 3) & 1)));
  g.a_frag = wm * 128 * kCpr;
  g.b_frag = (kSwiglu ? wn * 64 : wn * 128) * kCpr;

  // Output geometry: acc[i][j][4 q' + q] is row (lane & 31) of row block i and
  // column 8 q' + 4 (lane / 32) + q of weight block j; after pairing lanes l
  // and l + 32 a lane holds 8 consecutive columns of one row.
  constexpr int kStores = 4 * (kSwiglu ? 2 : 4) * 2;   // 16-byte stores per lane per tile
  static_assert(kPieces + kStores <= 63, "vmcnt range");

  // The k-tile sequence runs through this block's tiles; the refills fetch
  // from this tile (s0) or the next two (s1, s2; two ahead only when
  // nk == 2). Past the block's last tile they re-read that tile: in bounds,
  // never used.
  const int last = pos + ((total - 1 - pos) / G) * G;
  auto src_of = [&](int L) {
    return tile_src<kSwiglu, kGather>(
        a, tile_info<kOutCols>(a, pre, cnt_s, off_s, total_m, NT, min(L, last)), I, wave, lane);
  };
  TileInfo t = tile_info<kOutCols>(a, pre, cnt_s, off_s, total_m, NT, pos);
  TileSrc<kGather> s0 = tile_src<kSwiglu, kGather>(a, t, I, wave, lane);
  TileSrc<kGather> s1 = src_of(pos + G), s2 = src_of(pos + 2 * G);
  // k-tile q of the sequence starting at the current tile, q < 2 nk + 2
  auto pick = [&](int q, int& kq) -> TileSrc<kGather> {
    if (q < nk) {
      kq = q;
      return s0;
    }
    if (q < 2 * nk) {
      kq = q - nk;
      return s1;
    }
    kq = q - 2 * nk;
    return s2;
  };

  // reduce folded into GEMM2 (rows of received rows with one local slot go to
  // y): the slots of this lane's four rows of the current tile. Loaded ahead
  // of the operand loads so that the first use waits for none of them.
  constexpr bool fused = kFused;
  int slot_c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm * 128 + i * 32 + (lane & 31);
    slot_c[i] = (fused && row < t.rows_valid) ? a.dst[t.row0 + row] : -1;
  }

  Regs r0, r1;
  {
    int k0, k1, k2;
    const TileSrc<kGather> q0 = pick(0, k0), q1 = pick(1, k1), q2 = pick(2, k2);
#pragma unroll
    for (int j = 0; j < kPieces; ++j) dma_a<0>(g, q0, k0, j);
#pragma unroll
    for (int j = 0; j < kPieces; ++j) dma_a<1>(g, q1, k1, j);
#pragma unroll
    for (int j = 0; j < kPieces; ++j) r0.v[j] = load_b(q0, k0, j);
#pragma unroll
    for (int j = 0; j < kPieces; ++j) r1.v[j] = load_b(q1, k1, j);
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      write_b<0>(g, r0.v[j], j);
      r0.v[j] = load_b(q2, k2, j);
      __builtin_amdgcn_sched_barrier(0);   // write before reload
    }
    // stage 0 whole; r1 holds k-tile 1's weights (written to stage 1 in step
    // 0), r0 k-tile 2's; k-tile 1's activations may stay in flight
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * kPieces, true));
    lds_barrier();
  }
  Frags f;
  read_frags<0, 0, kSwiglu>(f, g, 0);

  // Whether the next tile's first step may leave this tile's kStores output
  // stores in flight. vmcnt counts in issue order, so "at most kPieces +
  // kStores outstanding" covers the activation DMA issued before the stores
  // only if all kStores were issued after it; the fused stores skip rows past
  // the segment, so after a partial fused tile the first step waits for the
  // stores as well.
  bool stores_in_flight = false;
#pragma clang loop unroll(disable)
  for (int L = pos; L < total; L += G) {
    {
      // Accumulators start at zero through an MFMA with zero operands: the
      // result lands in accumulation registers directly.
      bf16x8 zf;
      int zero = 0;
      asm volatile("" : "+v"(zero));
#pragma unroll
      for (int q = 0; q < 8; ++q) zf[q] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(zero));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          f.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zf, zf, floatx16{}, 0, 0, 0);
    }

    // Stages alternate with the k-tile's parity (nk is even). Step kt writes
    // the weights of k-tile kt + 1 from one register set and reloads it with
    // k-tile kt + 3, waits for the activations of k-tile kt + 1 (issued one
    // step earlier; after the previous tile's output stores for kt == 0) and
    // sends the activations of k-tile kt + 2 to its own stage.
    // (a do-while: nk >= 2, and no zero-trip path for the accumulators; not
    // peeled or unrolled, so there is one copy of the step code)
    // reduce folded into GEMM2: the weights of this tile's rows (their slots
    // were loaded one tile earlier) and the slots of the next tile's, so that
    // neither load is waited for before its use
    float ywt[4];
    int slot_n[4];
    if (fused) {
      const bool more = L + G < total;
      const TileInfo tn = tile_info<kOutCols>(a, pre, cnt_s, off_s, total_m, NT, more ? L + G : L);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ywt[i] = (slot_c[i] >= 0 && a.wts) ? a.wts[slot_c[i]] : 1.0f;
        const int row = wm * 128 + i * 32 + (lane & 31);
        slot_n[i] = (more && row < tn.rows_valid) ? a.dst[tn.row0 + row] : -1;
      }
    }

    bool after_stores = stores_in_flight;
    int kt = 0;
    // Steady state: while every DMA and weight load of the two steps reads
    // the current tile (k-tile kt + 4 < nk), the sources are fixed and the
    // loop selects nothing between tiles; the last steps take the general
    // form below.
#pragma clang loop unroll(disable)
    while (kt + 4 < nk) {
      ring_step<0, kSwiglu, kStores>(f, g, r1, after_stores, s0, kt + 2, s0, kt + 3);
      after_stores = false;
      ring_step<1, kSwiglu, kStores>(f, g, r0, false, s0, kt + 3, s0, kt + 4);
      kt += 2;
    }
#pragma clang loop unroll(disable)
    do {
      int dk, lk;
      {
        const TileSrc<kGather> d = pick(kt + 2, dk), l = pick(kt + 3, lk);
        ring_step<0, kSwiglu, kStores>(f, g, r1, after_stores, d, dk, l, lk);
      }
      after_stores = false;
      {
        const TileSrc<kGather> d = pick(kt + 3, dk), l = pick(kt + 4, lk);
        ring_step<1, kSwiglu, kStores>(f, g, r0, false, d, dk, l, lk);
      }
      kt += 2;
    } while (kt < nk);

    // The accumulators stay in accumulation registers up to their block's
    // turn in the epilogue.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(f.acc[i][j]));

    // Epilogue: bf16 (SwiGLU for the up projection) straight to global memory
    // with buffer stores whose range check drops rows past the segment.
    const uint64_t out_left = static_cast<uint64_t>(t.rows_valid) * a.Nc * 2;
    const __amdgpu_buffer_rsrc_t rC = __builtin_amdgcn_make_buffer_rsrc(
        Cb + static_cast<int64_t>(t.row0) * a.Nc, 0, static_cast<int>(out_left), kBufferFlags);
    const int hi = lane >> 5;
    // reduce folded into GEMM2: each of this lane's four rows goes to its
    // received row of y (one local slot) or to O; rows past the segment store
    // nothing
    uint16_t* drow[4];
    bool to_y[4], rvalid[4];
    float yadd[4];
    if (fused) {
      uint16_t* __restrict__ Yb = static_cast<uint16_t*>(a.y);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lrow = wm * 128 + i * 32 + (lane & 31);
        to_y[i] = slot_c[i] >= 0;
        yadd[i] = to_y[i] ? 0.0f : -0.0f;
        rvalid[i] = lrow < t.rows_valid;
        drow[i] = to_y[i] ? Yb + static_cast<int64_t>(slot_c[i] / a.K) * a.Nc
                          : Cb + static_cast<int64_t>(t.row0 + lrow) * a.Nc;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t row_off = static_cast<uint32_t>(wm * 128 + i * 32 + (lane & 31)) * a.Nc;
#pragma unroll
      for (int j = 0; j < (kSwiglu ? 2 : 4); ++j) {
        // Copy this block's accumulators to ordinary registers here and only
        // here (the empty asm pins the copy), so that the compiler does not
        // move the whole tile's accumulators out at once while the register
        // stages are live.
        floatx16 xg = f.acc[i][j];
        asm volatile("" : "+v"(xg));
        floatx16 xu = xg;
        if (kSwiglu) {
          xu = f.acc[i][j + 2];
          asm volatile("" : "+v"(xu));
        }
        uint32_t d[4][2];   // [column group q'][pair]: bf16 pairs of 4 columns
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int v0 = 4 * qq + 2 * h2, v1 = v0 + 1;
            float x0, x1;
            if (kSwiglu) {
              x0 = silu_mul(xg[v0], xu[v0]);
              x1 = silu_mul(xg[v1], xu[v1]);
            } else {
              x0 = xg[v0];
              x1 = xg[v1];
            }
            d[qq][h2] = pack_bf16x2_hw(x0, x1);
          }
        }
        const int colj = t.n0 + (kSwiglu ? wn * 64 : wn * 128) + j * 32;
#pragma unroll
        for (int qq = 0; qq < 4; qq += 2) {
          // lanes < 32 gather columns 8 qq + [0, 8), lanes >= 32 8 (qq+1) + [0, 8)
          const auto s0 = __builtin_amdgcn_permlane32_swap(d[qq][0], d[qq + 1][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(d[qq][1], d[qq + 1][1], false, false);
          const u32x4 out = u32x4{s0[0], s1[0], s0[1], s1[1]};
          const uint32_t col = colj + 8 * (qq + hi);
          if (!fused) {
            __builtin_amdgcn_raw_buffer_store_b128(out, rC, (row_off + col) * 2, 0, 0);
          } else {
            // a row of a received row with one local slot goes to y exactly
            // as the reduce writes it: fma(w, bf16 output, +0) in fp32,
            // rounded once (the +0 start of the reduce's sum decides the sign
            // of zero); the other rows go to O. One store either way, through
            // a per-lane address; rows past the segment store nothing. A row
            // to O takes the same arithmetic with w = 1 and the addend -0,
            // which returns its bf16 value unchanged (fma(1, v, -0) = v for
            // every v, zeros of both signs included), so there is no select
            // per value.
            u32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = pack_bf16x2_hw(
                  __builtin_fmaf(ywt[i], __uint_as_float(out[e] << 16), yadd[i]),
                  __builtin_fmaf(ywt[i], __uint_as_float(out[e] & 0xffff0000u), yadd[i]));
            if (rvalid[i]) *reinterpret_cast<u32x4*>(drow[i] + col) = v;
          }
        }
        // one weight block at a time: the register stages stay live here
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    stores_in_flight = !fused || t.rows_valid == BM;
    if (fused) {
#pragma unroll
      for (int i = 0; i < 4; ++i) slot_c[i] = slot_n[i];
    }
    if (L + G < total) t = tile_info<kOutCols>(a, pre, cnt_s, off_s, total_m, NT, L + G);
    s0 = s1;
    s1 = s2;
    s2 = src_of(L + 3 * G);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0, true));   // loads and DMA past the last tile
}

// Tiles begin + slot, begin + slot + nslots, ... below end of one GEMM, for
// this block; GEMM2 with a.dst takes the fused epilogue (one branch per
// launch, not per store).
template <bool kSwiglu, bool kGather>
__device__ __forceinline__ void gemm_tiles(const GemmArgs& a, int I, const int* pre,
                                           const int* cnt_s, const int* off_s, int total_m,
                                           int begin, int end, int slot, int nslots) {
  if constexpr (kSwiglu) {
    gemm_tiles_impl<true, kGather, false>(a, I, pre, cnt_s, off_s, total_m, begin, end, slot,
                                          nslots);
  } else {
    if (a.dst != nullptr)
      gemm_tiles_impl<false, kGather, true>(a, I, pre, cnt_s, off_s, total_m, begin, end, slot,
                                            nslots);
    else
      gemm_tiles_impl<false, kGather, false>(a, I, pre, cnt_s, off_s, total_m, begin, end, slot,
                                             nslots);
  }
}
#endif  // __HIP_DEVICE_COMPILE__

enum { kPartAll = 0, kPartWholeRounds = 1, kPartRest = 2 };

// One GEMM: every tile (kPartAll), GEMM1's whole rounds (kPartWholeRounds,
// launch 1 above) or GEMM2's tiles from n2 on (kPartRest, launch 3; g_split
// is launch 2's grid).
template <bool kSwiglu, bool kGather>
__global__ __launch_bounds__(kThreads) void gemm_tiled(GemmArgs a, int I, int part, int g_split) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ int pre[kMaxE + 1];
  __shared__ int tmp[kWavesT];
  __shared__ int cnt_s[kMaxE], off_s[kMaxE];
  const int total_m = gemm_prologue(a, pre, tmp, cnt_s, off_s);
  if (total_m < 0) return;
  constexpr int kOutCols = kSwiglu ? BN / 2 : BN;
  const int NT = (a.Nc + kOutCols - 1) / kOutCols;
  const int total = total_m * NT;
  if (total == 0) return;
  int begin = 0, end = total;
  if (part == kPartWholeRounds) end = total / static_cast<int>(gridDim.x) * static_cast<int>(gridDim.x);
  if (part == kPartRest)   // GEMM2: Kd = I, Nc = H
    begin = early_down_tiles(total_m, (a.Kd + BN / 2 - 1) / (BN / 2), NT, a.Nc / a.Kd, g_split);
  gemm_tiles<kSwiglu, kGather>(a, I, pre, cnt_s, off_s, total_m, begin, end, blockIdx.x,
                               gridDim.x);
#endif  // __HIP_DEVICE_COMPILE__
}

// Launch 2 above: GEMM1's last round on the first blocks, early GEMM2 tiles
// on the others (g1 and g2 share the plan's counts and mode).
//
// y may alias x. Early GEMM2 tiles write y only for received rows with one
// local slot, and that slot lies in an m-tile GEMM1 has already finished, so
// no GEMM1 tile of this launch reads such a row as one of its own; rows
// past a segment are not read at all (their DMA offset lies past x).
template <bool kGather>
__global__ __launch_bounds__(kThreads) void gemm_hybrid(GemmArgs g1, GemmArgs g2, int I) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ int pre[kMaxE + 1];
  __shared__ int tmp[kWavesT];
  __shared__ int cnt_s[kMaxE], off_s[kMaxE];
  const int total_m = gemm_prologue(g1, pre, tmp, cnt_s, off_s);
  if (total_m < 0) return;
  const int NT1 = (g1.Nc + BN / 2 - 1) / (BN / 2), NT2 = (g2.Nc + BN - 1) / BN;
  const int G = gridDim.x;
  const int total1 = total_m * NT1;
  const int R1 = total1 / G * G;
  const int tail = total1 - R1;
  if (static_cast<int>(blockIdx.x) < tail) {
    gemm_tiles<true, kGather>(g1, I, pre, cnt_s, off_s, total_m, R1, total1, blockIdx.x, tail);
  } else {
    const int n2 = early_down_tiles(total_m, NT1, NT2, g1.Kd / g2.Kd, G);
    gemm_tiles<false, false>(g2, I, pre, cnt_s, off_s, total_m, 0, n2, blockIdx.x - tail,
                             G - tail);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// --------------------------------------------------------------------------
// Weight-streaming kernel (bf16, experts with few rows)
// --------------------------------------------------------------------------
// The experts the streaming and decode kernels take (every non-empty one the
// mode streams),
// in expert order. With at most 64 experts every wave finds them on its own:
// lane e holds expert e's count and offset, a ballot marks the eligible
// ones, and the q-th is the set bit with q set bits below it (no LDS, no
// barrier before the first weight load). With more, the block-wide prefix
// and LDS tables.
struct StreamExperts {
  int n;                  // eligible experts
  bool wave;              // the wave form (E <= 64)
  uint64_t mask;          // wave form: the eligible experts' lanes
  int cnt_l, off_l;       // wave form: this lane's expert's count and offset
  __device__ __forceinline__ void get(int q, const int* list, const int* cnt_s,
                                      const int* off_s, int& e, int& cnt, int& off) const {
    if (wave) {
      const uint64_t hit =
          __ballot(((mask >> __lane_id()) & 1) && popc_below(mask) == q);
      e = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      cnt = __shfl(cnt_l, e, kWave);
      off = __shfl(off_l, e, kWave);
    } else {
      e = list[q];
      cnt = cnt_s[e];
      off = off_s[e];
    }
  }
};

template <int kBlock>
__device__ __forceinline__ StreamExperts stream_experts(const GemmArgs& a, int* pre, int* tmp,
                                                        int* list, int* cnt_s, int* off_s) {
  StreamExperts ex{};
  const int mode = a.mode;
  if (a.E <= kWave) {
    const int lane = __lane_id();
    const int e = min(lane, a.E - 1);
    const int c = a.counts[e], o = a.offsets[e];
    ex.wave = true;
    ex.mask = __ballot(lane < a.E && c > 0 && goes_to_stream(c, mode));
    ex.n = __popcll(ex.mask);
    ex.cnt_l = c;
    ex.off_l = o;
    return ex;
  }
  // the counts and offsets, loaded together with the prefix's
  int offv[kMaxE / kBlock], cntv[kMaxE / kBlock];
#pragma unroll
  for (int j = 0; j < kMaxE / kBlock; ++j) {
    const int e = min(static_cast<int>(threadIdx.x) + j * kBlock, a.E - 1);
    offv[j] = j * kBlock < a.E ? a.offsets[e] : 0;
    cntv[j] = j * kBlock < a.E ? a.counts[e] : 0;
  }
  ex.wave = false;
  ex.n = expert_prefix<kBlock>(a.counts, a.E, [mode](int c) {
    return (c > 0 && goes_to_stream(c, mode)) ? 1 : 0;
  }, pre, tmp);
#pragma unroll
  for (int j = 0; j < kMaxE / kBlock; ++j) {
    const int e = threadIdx.x + j * kBlock;
    if (e < a.E) {
      if (pre[e + 1] > pre[e]) list[pre[e]] = e;
      cnt_s[e] = cntv[j];
      off_s[e] = offv[j];
    }
  }
  __syncthreads();
  return ex;
}

constexpr int kStreamU = 8;  // k32 blocks per unrolled step

// This wave's k32 blocks [kb0, kb1) of one token group: NQ groups of 16 rows
// (the second only when the group has more than 16 rows, so that a decode
// group issues no loads for it). MFMA j of a step takes k-block kb + j: lane
// group g holds its 8 elements g * 8 .. g * 8 + 7, so one load instruction
// reads 64 contiguous bytes of each of 16 rows (4 lanes per row).
template <int NQ>
__device__ __forceinline__ void stream_kloop(const uint16_t* __restrict__ wp,
                                             const uint16_t* const (&xp)[2], const bool (&xv)[2],
                                             int kb0, int kb1, int g, floatx4 (&acc)[2]) {
  int kb = kb0;
  for (; kb + kStreamU <= kb1; kb += kStreamU) {
    const int k = kb * 32 + g * 8;
    u32x4 wa[kStreamU], xb[NQ][kStreamU];
#pragma unroll
    for (int j = 0; j < kStreamU; ++j) wa[j] = *reinterpret_cast<const u32x4*>(wp + k + j * 32);
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int j = 0; j < kStreamU; ++j)
        xb[q][j] = xv[q] ? *reinterpret_cast<const u32x4*>(xp[q] + k + j * 32)
                         : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kStreamU; ++j)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, wa[j]), __builtin_bit_cast(bf16x8, xb[q][j]), acc[q],
            0, 0, 0);
  }
  for (; kb < kb1; ++kb) {
    const int k = kb * 32 + g * 8;
    const u32x4 wa = *reinterpret_cast<const u32x4*>(wp + k);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const u32x4 xb = xv[q] ? *reinterpret_cast<const u32x4*>(xp[q] + k) : u32x4{0, 0, 0, 0};
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, wa), __builtin_bit_cast(bf16x8, xb), acc[q], 0, 0, 0);
    }
  }
}

template <bool kSwiglu>
__global__ __launch_bounds__(kThreads) void gemm_stream(GemmArgs a, int I) {
  __shared__ int pre[kMaxE + 1];
  __shared__ int list[kMaxE];
  __shared__ int cnt_s[kMaxE], off_s[kMaxE];
  __shared__ int tmp[kThreads / kWave];
  __shared__ floatx4 red[kThreads / kWave][2][kWave];

  // the experts' segment offsets, loaded with the counts (one wait; indices
  // clamped so that the loads are unconditional); a launch for which the
  // route scan counted no expert (a.n_take) exits before the prefix
  const int take = *a.n_take;
  // take experts give take * (units per expert) units, one per block in
  // turn: a block past them has none (the grid is sized for all E experts)
  if (static_cast<int>(blockIdx.x) >= take * ((a.Nc + (kSwiglu ? 8 : 16) - 1) / (kSwiglu ? 8 : 16)))
    return;
  const StreamExperts ex = stream_experts<kThreads>(a, pre, tmp, list, cnt_s, off_s);
  const int n_elig = ex.n;
  if (n_elig == 0) return;

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

  // Gathered A: the ids of this lane's rows (q * 16 + arow) of unit u's first
  // token group, loaded one unit ahead so that a unit starts with its rows
  // known.
  auto ids_of = [&](int u, int (&id)[2]) {
    id[0] = id[1] = 0;
    if (u >= total || !a.gather) return;
    int e, cnt, off;
    ex.get(u / upe, list, cnt_s, off_s, e, cnt, off);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int t = q * 16 + arow;
      if (t < cnt) id[q] = a.gather[off + t];
    }
  };
  int id_next[2];
  ids_of(blockIdx.x, id_next);
  for (int u = blockIdx.x; u < total; u += gridDim.x) {
    int e, cnt, off;
    ex.get(u / upe, list, cnt_s, off_s, e, cnt, off);
    const int c = u % upe;
    const int id0[2] = {id_next[0], id_next[1]};
    ids_of(u + static_cast<int>(gridDim.x), id_next);
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
        const int r = off + (xv[q] ? tok : 0);
        const int row = !a.gather ? r : tb == 0 ? id0[q] : a.gather[r];
        xp[q] = Ab + static_cast<int64_t>(row) * Kd;
      }

      floatx4 acc[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
      if (cnt - tb > 16) stream_kloop<2>(wp, xp, xv, kb0, kb1, g, acc);
      else stream_kloop<1>(wp, xp, xv, kb0, kb1, g, acc);
      red[wave][0][lane] = acc[0];
      red[wave][1][lane] = acc[1];
      __syncthreads();
      if (wave == 0) {
        // lane (g, r) holds output columns 4 g .. 4 g + 3 of the unit (the
        // weight rows) for token tb + 16 q + r; with the next four columns
        // from lane + 16, lanes of even g store 8 columns with one 16-byte
        // store (the unit's columns lie inside the row: I % 128 == 0,
        // H % 256 == 0)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int tok = tb + q * 16 + (lane & 15);
          floatx4 s = red[0][q][lane];
#pragma unroll
          for (int w = 1; w < kThreads / kWave; ++w) s += red[w][q][lane];
          uint32_t p0, p1;
          if (kSwiglu) {
            // lanes 0..31 hold gate rows, lanes 32..63 the matching up rows
            floatx4 up = red[0][q][lane ^ 32];
#pragma unroll
            for (int w = 1; w < kThreads / kWave; ++w) up += red[w][q][lane ^ 32];
            p0 = pack_bf16x2(silu_mul(s[0], up[0]), silu_mul(s[1], up[1]));
            p1 = pack_bf16x2(silu_mul(s[2], up[2]), silu_mul(s[3], up[3]));
          } else {
            p0 = pack_bf16x2(s[0], s[1]);
            p1 = pack_bf16x2(s[2], s[3]);
          }
          const uint32_t n0 = __shfl_down(p0, 16, kWave), n1 = __shfl_down(p1, 16, kWave);
          const bool st = kSwiglu ? g == 0 : (g & 1) == 0;
          const int col = kSwiglu ? c * 8 : c * 16 + 4 * g;
          if (st && tok < cnt && col + 8 <= a.Nc)
            *reinterpret_cast<u32x4*>(Cb + static_cast<int64_t>(off + tok) * a.Nc + col) =
                u32x4{p0, p1, n0, n1};
        }
      }
      __syncthreads();
    }
  }
}

// --------------------------------------------------------------------------
// Decode kernel (bf16; a batch of at most kStreamMaxRows expanded rows)
// --------------------------------------------------------------------------
// One decode step streams each active expert's weights once against a row or
// a few: its time is the read latency of the weights more than their
// bandwidth, and there are few units (one expert's 2I / 8 or H / 16), about
// one per CU. Units as in gemm_stream, the reduction split over kDecWaves
// waves; a wave issues every load of its share (kDecB k32 blocks at a time)
// and waits once, so a unit's weight bytes are in flight together. Token
// rows go in groups of 16, one after another (a decode expert rarely has
// more than 16).
constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * kWave;


// kDecB: k32 blocks per chunk (8 or 16, the launch picks the one that fits a
// wave's share with the fewest spare loads).
template <bool kSwiglu, int kDecB>
__global__ __launch_bounds__(kDecThreads) void gemm_decode(GemmArgs a, int I) {
  __shared__ int pre[kMaxE + 1];
  __shared__ int list[kMaxE];
  __shared__ int cnt_s[kMaxE], off_s[kMaxE];
  __shared__ int tmp[kDecWaves];
  __shared__ floatx4 red[kDecWaves][kWave];

  const StreamExperts ex = stream_experts<kDecThreads>(a, pre, tmp, list, cnt_s, off_s);
  const int n_elig = ex.n;
  if (n_elig == 0) return;

  const int cols = kSwiglu ? 8 : 16;               // outputs per unit
  const int upe = (a.Nc + cols - 1) / cols;        // units per expert
  const int total = n_elig * upe;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;                         // k group of the lane
  const int arow = lane & 15;                      // operand row of the lane
  const int Kd = a.Kd;
  const int nk32 = Kd / 32;
  const int kb0 = wave * nk32 / kDecWaves, kb1 = (wave + 1) * nk32 / kDecWaves;
  const int64_t Nb = kSwiglu ? 2 * static_cast<int64_t>(I) : a.Nc;
  const uint16_t* __restrict__ Ab = static_cast<const uint16_t*>(a.A);
  const uint16_t* __restrict__ Bb = static_cast<const uint16_t*>(a.B);
  uint16_t* __restrict__ Cb = static_cast<uint16_t*>(a.C);

  for (int u = blockIdx.x; u < total; u += gridDim.x) {
    int e, cnt, off;
    ex.get(u / upe, list, cnt_s, off_s, e, cnt, off);
    const int c = u % upe;
    int64_t wrow;
    if (kSwiglu) {
      const int col = min(c * 8 + (arow & 7), I - 1);
      wrow = arow < 8 ? col : I + col;
    } else {
      wrow = min(c * 16 + arow, a.Nc - 1);
    }
    const uint16_t* wp = Bb + (static_cast<int64_t>(e) * Nb + wrow) * Kd + g * 8;

    for (int tb = 0; tb < cnt; tb += 16) {
      const int tok = tb + arow;
      const bool xv = tok < cnt;
      const int r = off + (xv ? tok : 0);
      const int row = a.gather ? a.gather[r] : r;
      floatx4 acc = {0, 0, 0, 0};
      for (int kb = kb0; kb < kb1; kb += kDecB) {
        // every load of the chunk first, then one wait. The weight loads are
        // unconditional (blocks past the share re-read its last block, and
        // their MFMAs are skipped), so the compiler can count them and wait
        // for the row id below without waiting for them.
        u32x4 wa[kDecB], xb[kDecB];
#pragma unroll
        for (int j = 0; j < kDecB; ++j)
          wa[j] = *reinterpret_cast<const u32x4*>(wp + min(kb + j, kb1 - 1) * 32);
        // the token row's id is used only after the weight loads are out (the
        // empty asm takes it here and keeps the loads before it), so its
        // gather overlaps the weights' latency
        int rr = row;
        asm volatile("" : "+v"(rr) : : "memory");
        const uint16_t* xp = Ab + static_cast<int64_t>(rr) * Kd + g * 8;
#pragma unroll
        for (int j = 0; j < kDecB; ++j)
          if (kb + j < kb1)
            xb[j] = xv ? *reinterpret_cast<const u32x4*>(xp + (kb + j) * 32) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < kDecB; ++j)
          if (kb + j < kb1)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wa[j]),
                                                          __builtin_bit_cast(bf16x8, xb[j]), acc,
                                                          0, 0, 0);
      }
      red[wave][lane] = acc;
      __syncthreads();
      if (wave == 0) {
        // the waves' partial sums in a fixed order; lane (g, r) holds output
        // columns 4 g .. 4 g + 3 of the unit for token tb + r, lane + 16 the
        // next four, and lanes of even g store 8 columns with one 16-byte
        // store (I % 128 == 0, H % 256 == 0)
        floatx4 s = red[0][lane];
#pragma unroll
        for (int w = 1; w < kDecWaves; ++w) s += red[w][lane];
        uint32_t p0, p1;
        if (kSwiglu) {
          // lanes 0..31 hold gate rows, lanes 32..63 the matching up rows
          floatx4 up = red[0][lane ^ 32];
#pragma unroll
          for (int w = 1; w < kDecWaves; ++w) up += red[w][lane ^ 32];
          p0 = pack_bf16x2(silu_mul(s[0], up[0]), silu_mul(s[1], up[1]));
          p1 = pack_bf16x2(silu_mul(s[2], up[2]), silu_mul(s[3], up[3]));
        } else {
          p0 = pack_bf16x2(s[0], s[1]);
          p1 = pack_bf16x2(s[2], s[3]);
        }
        const uint32_t n0 = __shfl_down(p0, 16, kWave), n1 = __shfl_down(p1, 16, kWave);
        const bool st = kSwiglu ? g == 0 : (g & 1) == 0;
        const int col = kSwiglu ? c * 8 : c * 16 + 4 * g;
        if (st && xv && col + 8 <= a.Nc)
          *reinterpret_cast<u32x4*>(Cb + static_cast<int64_t>(off + tok) * a.Nc + col) =
              u32x4{p0, p1, n0, n1};
      }
      __syncthreads();
    }
  }
}


// Decode GEMM2 with the weighted top-k reduce folded in (moe_forward on a
// decode batch: at most kStreamMaxRows expanded rows, so at most that many
// received rows and slots). One unit is 16 output columns of every row: the
// block computes them for each active expert in turn, exactly as gemm_decode
// does (same split of k over the waves, same fixed-order sum, the same bf16
// rounding of O), keeps the rounded values in LDS, and then sums each
// received row's local slots in slot order into y, as fma(w, o, acc) from
// +0 and rounded once, exactly as the reduce kernel does. No row of O goes to
// memory and the reduce needs no launch of its own; a received row with no
// local slot gets +0. Rows at or past n_rows count as absent, as in the
// reduce; a slot's weight is read only when the slot is local.
template <int kDecB>
__global__ __launch_bounds__(kDecThreads) void gemm_decode_y(GemmArgs a,
                                                             const int* __restrict__ row_map,
                                                             int64_t n_rows) {
  __shared__ int pre[kMaxE + 1];
  __shared__ int list[kMaxE];
  __shared__ int cnt_s[kMaxE], off_s[kMaxE];
  __shared__ int tmp[kDecWaves];
  __shared__ floatx4 red[kDecWaves][kWave];
  __shared__ uint32_t o_s[kStreamMaxRows][8];   // bf16 pairs: row r, columns 2 i, 2 i + 1
  __shared__ int map_s[kStreamMaxRows];
  __shared__ float w_s[kStreamMaxRows];

  const int tid = threadIdx.x;
  const int TK = static_cast<int>(a.T) * a.K;   // <= kStreamMaxRows
  int mv = -1;
  if (tid < TK) {
    mv = row_map[tid];
    if (mv >= n_rows) mv = -1;
  }
  const StreamExperts ex = stream_experts<kDecThreads>(a, pre, tmp, list, cnt_s, off_s);
  const int n_elig = ex.n;
  // (map_s is read only after the barrier that stores w_s)
  if (tid < TK) map_s[tid] = mv;
  // the local slots' weights: needed only after the first unit's MFMAs
  const float wv = (tid < TK && mv >= 0 && a.wts) ? a.wts[tid] : 1.0f;

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;                         // k group of the lane
  const int arow = lane & 15;                      // operand row of the lane
  const int Kd = a.Kd;
  const int nk32 = Kd / 32;
  const int kb0 = wave * nk32 / kDecWaves, kb1 = (wave + 1) * nk32 / kDecWaves;
  const int64_t Nb = a.Nc;
  const uint16_t* __restrict__ Ab = static_cast<const uint16_t*>(a.A);
  const uint16_t* __restrict__ Bb = static_cast<const uint16_t*>(a.B);
  uint16_t* __restrict__ Yb = static_cast<uint16_t*>(a.y);
  const int n_units = (a.Nc + 15) / 16;
  bool w_stored = false;

  for (int c = blockIdx.x; c < n_units; c += gridDim.x) {
    const int64_t wrow = min(c * 16 + arow, a.Nc - 1);
    for (int q = 0; q < n_elig; ++q) {
      int e, cnt, off;
      ex.get(q, list, cnt_s, off_s, e, cnt, off);
      const uint16_t* wp = Bb + (static_cast<int64_t>(e) * Nb + wrow) * Kd + g * 8;
      for (int tb = 0; tb < cnt; tb += 16) {
        const int tok = tb + arow;
        const bool xv = tok < cnt;
        const int r = off + (xv ? tok : 0);
        floatx4 acc = {0, 0, 0, 0};
        for (int kb = kb0; kb < kb1; kb += kDecB) {
          u32x4 wa[kDecB], xb[kDecB];
#pragma unroll
          for (int j = 0; j < kDecB; ++j)
            wa[j] = *reinterpret_cast<const u32x4*>(wp + min(kb + j, kb1 - 1) * 32);
          const uint16_t* xp = Ab + static_cast<int64_t>(r) * Kd + g * 8;
#pragma unroll
          for (int j = 0; j < kDecB; ++j)
            if (kb + j < kb1)
              xb[j] = xv ? *reinterpret_cast<const u32x4*>(xp + (kb + j) * 32) : u32x4{0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < kDecB; ++j)
            if (kb + j < kb1)
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wa[j]),
                                                            __builtin_bit_cast(bf16x8, xb[j]), acc,
                                                            0, 0, 0);
        }
        red[wave][lane] = acc;
        __syncthreads();
        if (wave == 0 && xv) {
          // lane (g, r): columns 4 g .. 4 g + 3 of the unit for row off + tok
          floatx4 sum = red[0][lane];
#pragma unroll
          for (int w = 1; w < kDecWaves; ++w) sum += red[w][lane];
          o_s[off + tok][2 * g] = pack_bf16x2(sum[0], sum[1]);
          o_s[off + tok][2 * g + 1] = pack_bf16x2(sum[2], sum[3]);
        }
        __syncthreads();
      }
    }
    if (!w_stored) {
      if (tid < TK) w_s[tid] = wv;
      w_stored = true;
      __syncthreads();
    }
    // the reduce: thread (t, column) of the unit
    const int t = tid >> 4, col = tid & 15;
    if (t < a.T && c * 16 + col < a.Nc) {
      float acc = 0.0f;
      for (int k = 0; k < a.K; ++k) {
        const int m = map_s[t * a.K + k];
        if (m >= 0) {
          const uint32_t pair = o_s[m][col >> 1];
          acc = fmaf(w_s[t * a.K + k], bf16_bits_to_f32((col & 1) ? (pair >> 16) : (pair & 0xffffu)),
                     acc);
        }
      }
      Yb[static_cast<int64_t>(t) * a.Nc + c * 16 + col] =
          static_cast<uint16_t>(pack_bf16x2(acc, 0.0f) & 0xffffu);
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------------------
// fp32 kernel: fp32 MFMA (v_mfma_f32_16x16x4_f32), one wave per 16-row x
// 16-output tile
// --------------------------------------------------------------------------
// A 16x16x4 MFMA takes from lane l the A element (row l % 16, k l / 16) and
// the B element (k l / 16, column l % 16), and leaves in lane l the outputs
// (rows 4 (l / 16) + 0..3, column l % 16). Here lane l loads four consecutive
// k of its row, k0 + 4 (l / 16) + 0..3, from the activation row and from the
// weight row(s); MFMA step s uses element s, so the four steps of a 16-k
// chunk cover k0 .. k0 + 15 once each. Activation rows past the segment,
// weight rows past the last output column and k past the end load as zero (no
// access); outputs are stored only for valid rows and columns. fp32 shapes are
// small (the tiny fp32 workload), so tiles are small for parallelism and
// operands come straight from global memory, eight chunks of loads ahead of
// their MFMAs.
constexpr int F_BM = 16, F_BN = 16, F_BK = 16;

template <bool kSwiglu>
__global__ __launch_bounds__(kThreads) void gemm_f32(GemmArgs a, int I) {
  __shared__ int pre[kMaxE + 1];
  __shared__ int tmp[kThreads / kWave];

  const int total_m = expert_prefix(a.counts, a.E, [](int c) {
    return c > 0 ? (c + F_BM - 1) / F_BM : 0;
  }, pre, tmp);
  const int NT = (a.Nc + F_BN - 1) / F_BN;
  const int total = total_m * NT;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int Kd = a.Kd;
  const bool vec = (Kd & 3) == 0;   // rows start 16-byte aligned: float4 loads
  const int64_t Nb = kSwiglu ? 2 * static_cast<int64_t>(I) : a.Nc;
  const float* __restrict__ Af = static_cast<const float*>(a.A);
  const float* __restrict__ Bf = static_cast<const float*>(a.B);
  float* __restrict__ Cf = static_cast<float*>(a.C);

  // four floats of row p at k .. k + 3, zero past Kd (p == nullptr: zero)
  auto load4 = [Kd, vec](const float* p, int k, float* v) {
    if (p && vec && k < Kd) {
      const floatx4 q = *reinterpret_cast<const floatx4*>(p + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = q[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (p && k + i < Kd) ? p[k + i] : 0.0f;
    }
  };

  for (int L = blockIdx.x * (kThreads / kWave) + wave; L < total;
       L += gridDim.x * (kThreads / kWave)) {
    const int gm = L / NT, nt = L % NT;
    const int e = find_expert(pre, a.E, gm);
    const int mt = gm - pre[e];
    const int row0 = a.offsets[e] + mt * F_BM;
    const int rows_valid = min(F_BM, a.counts[e] - mt * F_BM);
    const int col = nt * F_BN + lr;
    const bool cv = col < a.Nc;
    const float* we = Bf + static_cast<int64_t>(e) * Nb * Kd;
    // GEMM1 from the received rows: row r of the segment order is row
    // gather[r] of x
    const int arow = row0 + lr;
    const float* ap =
        lr < rows_valid ? Af + static_cast<int64_t>(a.gather ? a.gather[arow] : arow) * Kd
                        : nullptr;
    const float* gp = cv ? we + static_cast<int64_t>(col) * Kd : nullptr;
    const float* up = (kSwiglu && cv) ? we + static_cast<int64_t>(I + col) * Kd : nullptr;
    floatx4 accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
    constexpr int kChunks = 8;
    for (int k0 = 0; k0 < Kd; k0 += kChunks * F_BK) {
      float av[kChunks][4], gv[kChunks][4], uv[kChunks][4];
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const int k = k0 + c * F_BK + 4 * lq;
        load4(ap, k, av[c]);
        load4(gp, k, gv[c]);
        if (kSwiglu) load4(up, k, uv[c]);
      }
#pragma unroll
      for (int c = 0; c < kChunks; ++c)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          accg = __builtin_amdgcn_mfma_f32_16x16x4f32(av[c][st], gv[c][st], accg, 0, 0, 0);
          if (kSwiglu) accu = __builtin_amdgcn_mfma_f32_16x16x4f32(av[c][st], uv[c][st], accu, 0, 0, 0);
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 4 * lq + q;
      if (r < rows_valid && cv)
        Cf[static_cast<int64_t>(row0 + r) * a.Nc + col] =
            kSwiglu ? silu_mul(accg[q], accu[q]) : accg[q];
    }
  }
}


// --------------------------------------------------------------------------
// bf16 kernel for any H (a multiple of 8) and any I: the shapes whose output
// columns do not fill the tiled kernel's 256-column tiles (H % 256 or
// I % 128 non-zero). One wave per 32-column x 32-row output tile, operands
// straight from global memory (L2), v_mfma_f32_16x16x32_bf16.
// --------------------------------------------------------------------------
// A 16x16x32 MFMA takes from lane l eight consecutive k of A row l % 16 and of
// B column l % 16, k group l / 16, and leaves in lane l the outputs (rows
// 4 (l / 16) + 0..3, column l % 16). Here A is the weights (rows = output
// columns) and B the activations (columns = tokens), so a lane ends with four
// consecutive output columns of one token. Rows of the weights or tokens past
// their end and k past Kd load as zero; k runs in 32-wide steps, four per
// batch of loads. GEMM1 may read its rows through `gather`; GEMM2 may send a
// row with a fused slot (dst >= 0) to y as fma(w, bf16 output, +0), rounded
// once, exactly as the tiled kernel's fused epilogue does.
constexpr int G_BM = 32, G_BN = 32;

template <bool kSwiglu>
__global__ __launch_bounds__(kThreads) void gemm_any(GemmArgs a, int I) {
  __shared__ int pre[kMaxE + 1];
  __shared__ int tmp[kThreads / kWave];

  const int total_m = expert_prefix(a.counts, a.E, [](int c) {
    return c > 0 ? (c + G_BM - 1) / G_BM : 0;
  }, pre, tmp);
  const int NT = (a.Nc + G_BN - 1) / G_BN;
  const int total = total_m * NT;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int Kd = a.Kd;
  const bool vec = (Kd & 7) == 0;   // rows start 16-byte aligned
  const int64_t Nb = kSwiglu ? 2 * static_cast<int64_t>(I) : a.Nc;
  const uint16_t* __restrict__ Ab = static_cast<const uint16_t*>(a.A);
  const uint16_t* __restrict__ Bb = static_cast<const uint16_t*>(a.B);
  uint16_t* __restrict__ Cb = static_cast<uint16_t*>(a.C);
  uint16_t* __restrict__ Yb = static_cast<uint16_t*>(a.y);

  // eight bf16 of row p at k .. k + 7 (k a multiple of 8), zero past Kd
  // (p == nullptr: zero)
  auto load8 = [Kd, vec](const uint16_t* p, int k) -> u32x4 {
    if (p && vec && k < Kd) return *reinterpret_cast<const u32x4*>(p + k);
    u32x4 w = {0, 0, 0, 0};
    if (p) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = k + 2 * i < Kd ? p[k + 2 * i] : 0;
        const uint32_t hi = k + 2 * i + 1 < Kd ? p[k + 2 * i + 1] : 0;
        w[i] = lo | (hi << 16);
      }
    }
    return w;
  };
  auto mfma = [](u32x4 x, u32x4 y, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                   __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
  };

  for (int L = blockIdx.x * (kThreads / kWave) + wave; L < total;
       L += gridDim.x * (kThreads / kWave)) {
    const int gm = L / NT, nt = L % NT;
    const int e = find_expert(pre, a.E, gm);
    const int mt = gm - pre[e];
    const int row0 = a.offsets[e] + mt * G_BM;
    const int rows_valid = min(G_BM, a.counts[e] - mt * G_BM);
    const uint16_t* we = Bb + static_cast<int64_t>(e) * Nb * Kd;
    const uint16_t *tp[2], *gp[2], *up[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lr + 16 * h;
      const int src = r < rows_valid ? (a.gather ? a.gather[row0 + r] : row0 + r) : -1;
      tp[h] = src >= 0 ? Ab + static_cast<int64_t>(src) * Kd : nullptr;
      const int col = nt * G_BN + lr + 16 * h;
      gp[h] = col < a.Nc ? we + static_cast<int64_t>(col) * Kd : nullptr;
      up[h] = (kSwiglu && col < a.Nc) ? we + static_cast<int64_t>(I + col) * Kd : nullptr;
    }
    floatx4 accg[2][2], accu[2][2];   // [column half][token half]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) accg[i][j] = accu[i][j] = floatx4{0, 0, 0, 0};
    constexpr int kSteps = 4;
    for (int k0 = 0; k0 < Kd; k0 += kSteps * 32) {
      u32x4 tv[kSteps][2], gv[kSteps][2], uv[kSteps][2];
#pragma unroll
      for (int c = 0; c < kSteps; ++c) {
        const int k = k0 + c * 32 + 8 * lq;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          tv[c][h] = load8(tp[h], k);
          gv[c][h] = load8(gp[h], k);
          if (kSwiglu) uv[c][h] = load8(up[h], k);
        }
      }
#pragma unroll
      for (int c = 0; c < kSteps; ++c)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            accg[i][j] = mfma(gv[c][i], tv[c][j], accg[i][j]);
            if (kSwiglu) accu[i][j] = mfma(uv[c][i], tv[c][j], accu[i][j]);
          }
    }
    // lane (lr, lq) of block [i][j]: token row 16 j + lr, output columns
    // nt * 32 + 16 i + 4 lq + 0..3
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 16 * j + lr;
      if (r >= rows_valid) continue;
      const int slot = a.dst ? a.dst[row0 + r] : -1;
      const float wt = (slot >= 0 && a.wts) ? a.wts[slot] : 1.0f;
      uint16_t* orow = slot >= 0 ? Yb + static_cast<int64_t>(slot / a.K) * a.Nc
                                 : Cb + static_cast<int64_t>(row0 + r) * a.Nc;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int col = nt * G_BN + 16 * i + 4 * lq;
        uint32_t v[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float x0 = kSwiglu ? silu_mul(accg[i][j][2 * q], accu[i][j][2 * q]) : accg[i][j][2 * q];
          float x1 = kSwiglu ? silu_mul(accg[i][j][2 * q + 1], accu[i][j][2 * q + 1])
                             : accg[i][j][2 * q + 1];
          uint32_t b = pack_bf16x2_hw(x0, x1);
          if (slot >= 0)
            b = pack_bf16x2_hw(__builtin_fmaf(wt, __uint_as_float(b << 16), 0.0f),
                               __builtin_fmaf(wt, __uint_as_float(b & 0xffff0000u), 0.0f));
          v[q] = b;
        }
        if (col + 4 <= a.Nc && (a.Nc & 3) == 0) {
          *reinterpret_cast<uint2*>(orow + col) = uint2{v[0], v[1]};
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (col + q < a.Nc) orow[col + q] = static_cast<uint16_t>(v[q >> 1] >> (16 * (q & 1)));
        }
      }
    }
  }
}

}  // namespace

bool gemm_can_gather(const tr_moe_desc& d) {
  return d.dtype == TR_BF16 && d.T * d.H * 2 <= 0x7fffffffLL;
}

hipError_t grouped_gemm(const tr_moe_plan& p, const void* w1, const void* w2, int parts,
                        hipStream_t st, const void* x_gather, const float* w_fused,
                        void* y_fused, bool* y_done) {
  if (y_done) *y_done = false;
  const tr_moe_desc& d = p.d;
  if (d.T == 0) return hipSuccess;
  const int cus = device_cu_count();
  // A small batch in the automatic mode streams every expert (the route scan
  // assumed as much when it marked rows for the reduce folded into GEMM2;
  // at most kStreamMaxRows expanded rows no expert can have more anyway).
  int mode = kModeAuto;
  if (d.flags & TR_FLAG_GEMM_FORCE_TILED) mode = kModeTiled;
  else if (d.flags & TR_FLAG_GEMM_FORCE_STREAM) mode = kModeStream;
  else if (p.R_cap > kStreamMaxRows && p.R_cap <= kSmallBatchRows) mode = kModeStream;
  const int E = d.E;
  const int I = static_cast<int>(d.I);
  const bool up = parts & kGemmUp, down = parts & kGemmDown;
  const int64_t a_rows = p.R_cap + kRowPad;
  GemmArgs g1{p.Xe, w1, p.h, p.counts, p.offsets, E, static_cast<int>(d.H), I, mode, a_rows,
              nullptr, nullptr, nullptr, nullptr, d.K, d.T};
  if (x_gather) {
    // GEMM1 reads the received rows through the route table: no Xe
    g1.A = x_gather;
    g1.a_rows = d.T;
    g1.gather = p.row_src;
  }
  GemmArgs g2{p.h, w2, p.O, p.counts, p.offsets, E, I, static_cast<int>(d.H), mode, a_rows,
              nullptr, nullptr, nullptr, nullptr, d.K, d.T};
  if (y_fused && d.dtype == TR_BF16) {
    g2.dst = p.row_dst;
    g2.wts = w_fused;
    g2.y = y_fused;
  }
  hipError_t err;
  // the route scan's counts of the experts each bf16 kernel takes: a launch
  // that finds none exits after one load
  GemmArgs g1t = g1, g2t = g2, g1s = g1, g2s = g2;
  g1t.n_take = g2t.n_take = p.stats + 7;
  g1s.n_take = g2s.n_take = p.stats + 6;

  if (d.dtype == TR_F32) {
    // one tile per wave, four waves per block
    const int64_t tiles1 = (cdiv(p.R_cap, F_BM) + E) * cdiv(I, F_BN);
    const int64_t tiles2 = (cdiv(p.R_cap, F_BM) + E) * cdiv(d.H, F_BN);
    const int64_t b1 = cdiv(tiles1, kThreads / kWave), b2 = cdiv(tiles2, kThreads / kWave);
    const unsigned grid1 = static_cast<unsigned>(b1 < cus * 8 ? b1 : cus * 8);
    const unsigned grid2 = static_cast<unsigned>(b2 < cus * 8 ? b2 : cus * 8);
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

  // bf16 shapes whose output columns do not fill the tiled kernel's tiles:
  // the any-shape kernel for both GEMMs, one 32 x 32 tile per wave
  if (d.H % kColMultiple || d.I % (kColMultiple / 2)) {
    const int64_t tiles1 = (cdiv(p.R_cap, G_BM) + E) * cdiv(I, G_BN);
    const int64_t tiles2 = (cdiv(p.R_cap, G_BM) + E) * cdiv(d.H, G_BN);
    const int64_t b1 = cdiv(tiles1, kThreads / kWave), b2 = cdiv(tiles2, kThreads / kWave);
    const unsigned grid1 = static_cast<unsigned>(b1 < cus * 8 ? b1 : cus * 8);
    const unsigned grid2 = static_cast<unsigned>(b2 < cus * 8 ? b2 : cus * 8);
    if (up) {
      hipLaunchKernelGGL(gemm_any<true>, dim3(grid1), dim3(kThreads), 0, st, g1, I);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (down) {
      hipLaunchKernelGGL(gemm_any<false>, dim3(grid2), dim3(kThreads), 0, st, g2, I);
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
  // With at most kStreamMaxRows expanded rows no expert can reach the tiled
  // kernel in AUTO mode: skip its launch (decode batches).
  const bool tiled = mode == kModeTiled || (mode == kModeAuto && p.R_cap > kStreamMaxRows);
  // Both GEMMs with enough tiles for more than two rounds (by the bound
  // above): three launches, GEMM2 tiles filling GEMM1's last round (see
  // early_down_tiles). The whole-round and hybrid launches share one grid,
  // which the last one is told.
  const bool split = up && down && tiled && t1 > 2 * static_cast<int64_t>(cus);
  if (split) {
    const unsigned gsplit = gt1;
    if (g1.gather)
      hipLaunchKernelGGL((gemm_tiled<true, true>), dim3(gsplit), dim3(kThreads), 0, st, g1t, I,
                         static_cast<int>(kPartWholeRounds), 0);
    else
      hipLaunchKernelGGL((gemm_tiled<true, false>), dim3(gsplit), dim3(kThreads), 0, st, g1t, I,
                         static_cast<int>(kPartWholeRounds), 0);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (mode != kModeTiled) {
      hipLaunchKernelGGL(gemm_stream<true>, dim3(gs1), dim3(kThreads), 0, st, g1s, I);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (g1.gather)
      hipLaunchKernelGGL((gemm_hybrid<true>), dim3(gsplit), dim3(kThreads), 0, st, g1t, g2t, I);
    else
      hipLaunchKernelGGL((gemm_hybrid<false>), dim3(gsplit), dim3(kThreads), 0, st, g1t, g2t, I);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((gemm_tiled<false, false>), dim3(gt2), dim3(kThreads), 0, st, g2t, I,
                       static_cast<int>(kPartRest), static_cast<int>(gsplit));
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (mode != kModeTiled) {
      hipLaunchKernelGGL(gemm_stream<false>, dim3(gs2), dim3(kThreads), 0, st, g2s, I);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
  }
  if (up && tiled) {
    if (g1.gather)
      hipLaunchKernelGGL((gemm_tiled<true, true>), dim3(gt1), dim3(kThreads), 0, st, g1t, I,
                         static_cast<int>(kPartAll), 0);
    else
      hipLaunchKernelGGL((gemm_tiled<true, false>), dim3(gt1), dim3(kThreads), 0, st, g1t, I,
                         static_cast<int>(kPartAll), 0);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // A decode batch (AUTO mode, at most kStreamMaxRows expanded rows, so no
  // tiled experts): the latency-minded kernel, one block per unit up to one
  // per CU.
  const bool decode = mode == kModeAuto && p.R_cap <= kStreamMaxRows;
  const unsigned gd1 = static_cast<unsigned>(u1 < cus ? u1 : cus);
  const unsigned gd2 = static_cast<unsigned>(u2 < cus ? u2 : cus);
  // each wave's share of k32 blocks: chunks of 8 when it fits, else 16
  const bool dec8_up = cdiv(cdiv(d.H, 32), kDecWaves) <= 8;
  const bool dec8_down = cdiv(cdiv(I, 32), kDecWaves) <= 8;
  if (up && mode != kModeTiled) {
    if (decode && dec8_up)
      hipLaunchKernelGGL((gemm_decode<true, 8>), dim3(gd1), dim3(kDecThreads), 0, st, g1, I);
    else if (decode)
      hipLaunchKernelGGL((gemm_decode<true, 16>), dim3(gd1), dim3(kDecThreads), 0, st, g1, I);
    else
      hipLaunchKernelGGL(gemm_stream<true>, dim3(gs1), dim3(kThreads), 0, st, g1s, I);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (down && tiled) {
    hipLaunchKernelGGL((gemm_tiled<false, false>), dim3(gt2), dim3(kThreads), 0, st, g2t, I,
                       static_cast<int>(kPartAll), 0);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (down && mode != kModeTiled) {
    if (decode && y_done && g2.y) {
      // the reduce folded in: y complete after this launch
      const unsigned gy = static_cast<unsigned>(cdiv(d.H, 16) < cus ? cdiv(d.H, 16) : cus);
      if (dec8_down)
        hipLaunchKernelGGL((gemm_decode_y<8>), dim3(gy), dim3(kDecThreads), 0, st, g2,
                           p.row_map, p.R_cap);
      else
        hipLaunchKernelGGL((gemm_decode_y<16>), dim3(gy), dim3(kDecThreads), 0, st, g2,
                           p.row_map, p.R_cap);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      *y_done = true;
      return hipSuccess;
    }
    if (decode && dec8_down)
      hipLaunchKernelGGL((gemm_decode<false, 8>), dim3(gd2), dim3(kDecThreads), 0, st, g2, I);
    else if (decode)
      hipLaunchKernelGGL((gemm_decode<false, 16>), dim3(gd2), dim3(kDecThreads), 0, st, g2, I);
    else
      hipLaunchKernelGGL(gemm_stream<false>, dim3(gs2), dim3(kThreads), 0, st, g2s, I);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace tr
