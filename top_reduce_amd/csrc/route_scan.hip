// moe_route_scan: per-expert histogram, segment offsets and the stable maps
// between received slots (t, k) and expanded rows.
//
// DeepEP issue #48 ("How to apply MoE MLP to recv_x ... num_expert_per_rank >
// 1", answers): a grouped GEMM needs each token copied once per local expert,
// in expert-contiguous segments, and the reduction afterwards must find every
// copy again. Slot (t, k) is local when its id lies in [expert_begin,
// expert_begin + E); the others (-1 padding and other ranks' experts, DeepEP
// issue #760 repro) are skipped. Inside a segment rows follow the received
// order: token-major, then slot.
//
// Design (one GPU, no host sync):
//  - rows are cut into fixed blocks; kernel `route_count` writes each block's
//    per-expert counts (plus ignored slots and rows with a local route);
//  - kernel `route_scatter` has every block sum the partials into totals and
//    its own starting position per expert, then rank its slots with wave
//    ballots: lanes holding the same expert find each other by matching the
//    expert id bit by bit, their rank is a popcount of the lower peers, and
//    waves are chained in LDS. Positions never depend on atomic order, so the
//    maps are bit-exact and deterministic.
//  - the received rows that the fused GEMM2 epilogue does not complete
//    (tok_rest) are listed in row order: `route_count` also counts, per block,
//    the rows without exactly one local slot and, per expert, the rows whose
//    one local slot goes to it, so each block's first entry follows from the
//    same partial sums once the experts' totals are known.
//  - a small input runs as one block: up to 1024 slots a single-block
//    kernel with one slot per thread (decode batches), up to 2048 the
//    general scatter counting for itself; one launch instead of two.
//  - a DP-padded buffer (SGLang PR #6092: workers' batches padded to one
//    shape) names per block of rows how many carry tokens; the other rows are
//    treated as rows without a local slot, and their ids are never loaded.
#include "tr_device.h"
#include "tr_internal.h"

namespace tr {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
// A block keeps each of its slots' local expert and expanded row in LDS for
// the last phase when it has at most this many slots (else it re-reads them).
constexpr int kSlotCache = 2048;
constexpr int kMisc = 10;          // block-wide counters of the scatter kernel

template <typename IdxT>
__device__ __forceinline__ int local_of(IdxT id, int64_t eb, int E) {
  const int64_t e = static_cast<int64_t>(id) - eb;
  return (e >= 0 && e < E) ? static_cast<int>(e) : E;  // E: not local
}

// Whether received row r carries a token: every row without padding blocks
// (B == 0); else the first bc[j] rows of block j (B rows each), so a count
// above B means all of them and one at or below 0 none.
__device__ __forceinline__ bool carries(int64_t r, int B, const int* __restrict__ bc) {
  if (B == 0) return true;
  const int64_t j = static_cast<int>(r) / B;   // r < T < 2^31
  return r - j * B < bc[j];
}

// Per-block counts, kept in LDS and in each block's row of `hist`
// (hist_width(E) ints): [0, E) slots per local expert; then ignored slots,
// rows with at least one local slot, rows that carry a token, rows whose
// number of local slots is not one (rows that carry no token included); then
// [E + 4, 2 E + 4) rows whose only local slot goes to expert e.
__host__ __device__ constexpr int hist_width(int E) { return 2 * E + 4; }
enum { kIgn = 0, kLocalRows = 1, kCarry = 2, kNotOne = 3 };   // offsets past E

// Adds the slots and rows of rows [r0, r1) to cnt[0..hist_width(E)). Rows
// that do not carry a token count as rows without one local slot only.
// expert_of(s): the local expert of slot s of a carrying row, or E.
template <typename ExpertOf>
__device__ void count_rows(ExpertOf expert_of, int64_t r0, int64_t r1, int K, int E, int B,
                           const int* __restrict__ bc, int* cnt) {
  const int64_t s0 = r0 * K, s1 = r1 * K;
  for (int64_t base = s0; base < s1; base += kThreads) {
    const int64_t s = base + threadIdx.x;
    const bool in = s < s1 && (B == 0 || carries(static_cast<int>(s) / K, B, bc));
    const int e = in ? expert_of(s) : E;
    if (e < E) atomicAdd(&cnt[e], 1);
    const uint64_t ign = __ballot(in && e == E);
    if (lane_id() == 0 && ign) atomicAdd(&cnt[E + kIgn], __popcll(ign));
  }
  for (int64_t base = r0; base < r1; base += kThreads) {
    const int64_t r = base + threadIdx.x;
    const bool in = r < r1 && (B == 0 || carries(r, B, bc));
    int n = 0, e1 = E;
    if (in) {
#pragma unroll 8
      for (int k = 0; k < K; ++k) {
        const int e = expert_of(r * K + k);
        if (e < E) {
          ++n;
          e1 = e;
        }
      }
    }
    const uint64_t m = __ballot(n > 0);
    if (lane_id() == 0 && m) atomicAdd(&cnt[E + kLocalRows], __popcll(m));
    const uint64_t c = __ballot(in);
    if (lane_id() == 0 && c) atomicAdd(&cnt[E + kCarry], __popcll(c));
    const uint64_t no = __ballot(r < r1 && n != 1);
    if (lane_id() == 0 && no) atomicAdd(&cnt[E + kNotOne], __popcll(no));
    if (n == 1) atomicAdd(&cnt[E + 4 + e1], 1);
  }
}

template <typename IdxT>
__global__ __launch_bounds__(kThreads) void route_count(const IdxT* __restrict__ idx, int64_t T,
                                                        int K, int64_t eb, int E, int rpb, int B,
                                                        const int* __restrict__ bc,
                                                        int* __restrict__ hist) {
  extern __shared__ int cnt[];
  const int W = hist_width(E);
  for (int i = threadIdx.x; i < W; i += kThreads) cnt[i] = 0;
  __syncthreads();
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rpb;
  const int64_t r1 = r0 + rpb < T ? r0 + rpb : T;
  count_rows([&](int64_t s) { return local_of(idx[s], eb, E); }, r0, r1, K, E, B, bc, cnt);
  __syncthreads();
  for (int i = threadIdx.x; i < W; i += kThreads) hist[blockIdx.x * W + i] = cnt[i];
}

// Sum of v over the wave (all lanes receive it).
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

// kSelf: single block, counts its own rows instead of reading `hist`.
template <typename IdxT, bool kSelf>
__global__ __launch_bounds__(kThreads) void route_scatter(
    const IdxT* __restrict__ idx, int64_t T, int K, int64_t eb, int E, int rpb, int nblocks,
    int B, const int* __restrict__ bc, const int* __restrict__ hist, int* __restrict__ counts, int* __restrict__ offsets,
    int* __restrict__ row_map, int* __restrict__ row_src, int* __restrict__ row_k,
    int* __restrict__ stats, int* __restrict__ row_dst, int* __restrict__ tok_rest,
    int min_tiled) {
  extern __shared__ int sh[];
  const int W = hist_width(E);
  int* base = sh;                       // [E] first row of this block's slots per expert
  int* running = base + E;              // [E] rows taken so far by this block
  int* wcnt = running + E;              // [kWaves][E + 1] per-wave counts of a round
  int* cnt = wcnt + kWaves * (E + 1);   // [W] totals over the blocks (own counts: kSelf)
  int* tmp = cnt + W;                   // [kWaves] scan scratch
  int* misc = tmp + kWaves;             // [kMisc]
  int* slot_e = misc + kMisc;           // [kSlotCache] local expert of each slot (E: none)
  int* slot_row = slot_e + kSlotCache;  // [kSlotCache] its expanded row (-1: none)
  // misc: [0] empty experts, [1] ignored slots, [2] rows with a local slot,
  // [3] carrying rows, [4] rows without one local slot in earlier blocks,
  // [5] the same over all blocks, [6] / [7] rows whose one local slot goes
  // to a streamed expert, in earlier blocks / in all blocks, [8] / [9]
  // experts the streaming / the tiled GEMM takes

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rpb;
  const int64_t r1 = r0 + rpb < T ? r0 + rpb : T;

  int* prior = wcnt;                    // [E] phase 1 only; wcnt is zeroed after
  int* sprior = wcnt + E;               // [E] likewise: one-slot rows in earlier blocks
  for (int i = tid; i < W; i += kThreads) cnt[i] = 0;
  for (int i = tid; i < 2 * E; i += kThreads) prior[i] = 0;
  if (tid < kMisc) misc[tid] = 0;
  const int64_t s0 = r0 * K, s1 = r1 * K;
  const bool cache = s1 - s0 <= kSlotCache;
  // The local expert of each of this block's slots (E: none), kept in LDS
  // for the ranking and the last phase, and the other blocks' partial counts:
  // all loaded before the first barrier, so that they wait for memory once.
  // (The loads below are unconditional, with indices clamped into range and
  // the extra values masked afterwards, so that they all go out before the
  // first wait; a load under a per-lane condition would wait for its
  // predecessors first. Padding rows' ids are the exception: never read.)
  constexpr int kPer = kSlotCache / kThreads;
  int pe[kPer];
  IdxT pv[kPer] = {};   // raw ids (B == 0), converted once the other loads are out
  if (cache) {
    if (B == 0) {
      // clamped to the block's last slot; an empty block (T == 0) loads none
      if (s1 > s0) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int64_t s = s0 + tid + u * kThreads;
          pv[u] = idx[s < s1 ? s : s1 - 1];
        }
      }
    } else {
      // padding rows' ids are not read: each id load has its own condition,
      // and the ids are converted after the last load is out; the rows'
      // block counts are read first, all at once (rows clamped to the
      // block's last; an empty block (T == 0) reads none)
      int bcv[kPer] = {};
      if (s1 > s0) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int64_t s = s0 + tid + u * kThreads;
          bcv[u] = bc[static_cast<int>(s < s1 ? s : s1 - 1) / K / B];
        }
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int64_t s = s0 + tid + u * kThreads;
        const int r = static_cast<int>(s) / K;
        pe[u] = s < s1 && r - r / B * B < bcv[u] ? 1 : 0;
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        if (pe[u]) pv[u] = idx[s0 + tid + u * kThreads];
    }
  }
  // expert tid % E of blocks tid / E, + kThreads / E, ... (few enough experts
  // that a thread holds all of its blocks' counts in registers)
  constexpr int kHistPer = 32;
  const int lanes = E <= kThreads ? kThreads / E : 1;
  const bool hist_regs = !kSelf && E <= kThreads && cdiv(nblocks, lanes) <= kHistPer;
  int hc[kHistPer], hs[kHistPer];
  const int he = tid % E, hb0 = tid / E;
  if (hist_regs) {
    const int nper = static_cast<int>(cdiv(nblocks, lanes));   // uniform
#pragma unroll
    for (int u = 0; u < kHistPer; ++u) {
      const int b = min(hb0 + u * lanes, nblocks - 1);
      hc[u] = u < nper ? hist[b * W + he] : 0;
      hs[u] = u < nper ? hist[b * W + E + 4 + he] : 0;
    }
  }
  // block tid's row counts (nblocks <= kThreads)
  int h_not1 = 0, h_ign = 0, h_loc = 0, h_car = 0;
  if (!kSelf) {
    const int b = min(tid, nblocks - 1);
    h_not1 = hist[b * W + E + kNotOne];
    h_ign = hist[b * W + E + kIgn];
    h_loc = hist[b * W + E + kLocalRows];
    h_car = hist[b * W + E + kCarry];
    if (tid >= nblocks) h_not1 = h_ign = h_loc = h_car = 0;
  }
  if (cache) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const bool has = B == 0 ? s0 + tid + u * kThreads < s1 : pe[u] != 0;
      pe[u] = has ? local_of(pv[u], eb, E) : E;
      const int64_t s = s0 + tid + u * kThreads;
      if (s < s1) slot_e[s - s0] = pe[u];
    }
  }
  __syncthreads();
  if (kSelf) {
    // a single block counts its own slots: from the LDS slot table when it
    // has one (with padding blocks it also needs the rows' carrying state,
    // which the table does not keep)
    if (cache && B == 0)
      count_rows([&](int64_t s) { return slot_e[s - s0]; }, r0, r1, K, E, B, bc, cnt);
    else
      count_rows([&](int64_t s) { return local_of(idx[s], eb, E); }, r0, r1, K, E, B, bc, cnt);
  } else {
    if (hist_regs) {
      int all = 0, before = 0, sall = 0, sbefore = 0;
#pragma unroll
      for (int u = 0; u < kHistPer; ++u) {
        const int b = hb0 + u * lanes;
        if (hb0 < lanes && b < nblocks) {
          all += hc[u];
          sall += hs[u];
          if (b < static_cast<int>(blockIdx.x)) {
            before += hc[u];
            sbefore += hs[u];
          }
        }
      }
      if (all) atomicAdd(&cnt[he], all);
      if (before) atomicAdd(&prior[he], before);
      if (sall) atomicAdd(&cnt[E + 4 + he], sall);
      if (sbefore) atomicAdd(&sprior[he], sbefore);
    } else if (E <= kThreads) {
      // more blocks per thread: the same sums, 16 loads in flight at a time
      int all = 0, before = 0, sall = 0, sbefore = 0;
      if (hb0 < lanes) {
        for (int b = hb0; b < nblocks; b += 16 * lanes) {
          int c[16], cs[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int bu = min(b + u * lanes, nblocks - 1);
            c[u] = hist[bu * W + he];
            cs[u] = hist[bu * W + E + 4 + he];
          }
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int bu = b + u * lanes;
            if (bu < nblocks) {
              all += c[u];
              sall += cs[u];
              if (bu < static_cast<int>(blockIdx.x)) {
                before += c[u];
                sbefore += cs[u];
              }
            }
          }
        }
      }
      if (all) atomicAdd(&cnt[he], all);
      if (before) atomicAdd(&prior[he], before);
      if (sall) atomicAdd(&cnt[E + 4 + he], sall);
      if (sbefore) atomicAdd(&sprior[he], sbefore);
    } else {
      // many experts: all threads share the (block, expert) grid
      const int n = nblocks * E;
      for (int i = tid; i < n; i += kThreads) {
        const int b = i / E, e = i - b * E;
        const int c = hist[b * W + e], cs = hist[b * W + E + 4 + e];
        if (c) atomicAdd(&cnt[e], c);
        if (cs) atomicAdd(&cnt[E + 4 + e], cs);
        if (b < static_cast<int>(blockIdx.x)) {
          if (c) atomicAdd(&prior[e], c);
          if (cs) atomicAdd(&sprior[e], cs);
        }
      }
    }
    const int n1b = wave_sum(tid < static_cast<int>(blockIdx.x) ? h_not1 : 0);
    const int n1a = wave_sum(h_not1);
    // ignored slots, rows with a local slot and carrying rows: block 0's stats
    const int ig = wave_sum(h_ign), lo = wave_sum(h_loc), ca = wave_sum(h_car);
    if (lane_id() == 0) {
      if (n1b) atomicAdd(&misc[4], n1b);
      if (n1a) atomicAdd(&misc[5], n1a);
      if (ig) atomicAdd(&misc[1], ig);
      if (lo) atomicAdd(&misc[2], lo);
      if (ca) atomicAdd(&misc[3], ca);
    }
  }
  __syncthreads();

  // 1. totals per expert, this block's prior count, segment offsets, and the
  // tok_rest entries before this block's: rows without one local slot, and
  // one-slot rows of streamed experts (fewer than min_tiled routes).
  const int per = (E + kThreads - 1) / kThreads;  // experts per thread (<= 4)
  int tsum = 0, rest_before = 0, rest_all = 0;
  int tot[4], pri[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    tot[j] = 0;
    pri[j] = 0;
    const int e = tid * per + j;
    if (j < per && e < E) {
      tot[j] = cnt[e];
      pri[j] = kSelf ? 0 : prior[e];
      tsum += tot[j];
      if (tot[j] < min_tiled) {
        rest_before += kSelf ? 0 : sprior[e];
        rest_all += cnt[E + 4 + e];
      }
    }
  }
  rest_before = wave_sum(rest_before);
  rest_all = wave_sum(rest_all);
  __syncthreads();                      // prior[] read; wcnt becomes per-wave counts
  for (int i = tid; i < kWaves * (E + 1); i += kThreads) wcnt[i] = 0;
  if (lane_id() == 0) {
    if (rest_before) atomicAdd(&misc[6], rest_before);
    if (rest_all) atomicAdd(&misc[7], rest_all);
  }
  int R = 0;
  int off = block_exclusive_scan<kThreads>(tsum, tmp, &R);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * per + j;
    if (j < per && e < E) {
      base[e] = off + pri[j];
      running[e] = 0;
      if (blockIdx.x == 0) {
        counts[e] = tot[j];
        offsets[e] = off;
        if (tot[j] == 0) atomicAdd(&misc[0], 1);
        else atomicAdd(&misc[tot[j] < min_tiled ? 8 : 9], 1);
      }
      off += tot[j];
    }
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid == 0) {
    offsets[E] = R;
    stats[0] = R;
    stats[1] = kSelf ? cnt[E + kLocalRows] : misc[2];
    stats[2] = kSelf ? cnt[E + kIgn] : misc[1];
    stats[3] = misc[0];
    stats[4] = (kSelf ? cnt[E + kNotOne] : misc[5]) + misc[7];
    stats[5] = kSelf ? cnt[E + kCarry] : misc[3];
    stats[6] = misc[8];
    stats[7] = misc[9];
  }
  int rest_at = kSelf ? 0 : misc[4] + misc[6];

  // 2. stable ranks, one round of kThreads slots at a time.
  const int nbits = 32 - __clz(E);  // bits of the values 0..E
  for (int64_t rb = s0; rb < s1; rb += kThreads) {
    const int64_t s = rb + tid;
    const bool in = s < s1;
    const int e = !in ? E
                  : cache ? slot_e[s - s0]
                  : (B == 0 || carries(static_cast<int>(s) / K, B, bc)) ? local_of(idx[s], eb, E) : E;
    const bool valid = e < E;
    uint64_t peers = __ballot(1);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int rank = popc_below(peers);
    const bool leader = rank == 0;
    if (leader && valid) wcnt[wave * (E + 1) + e] = __popcll(peers);
    __syncthreads();
    int row = -1;
    if (valid) {
      int before = 0;
      for (int w = 0; w < wave; ++w) before += wcnt[w * (E + 1) + e];
      row = base[e] + running[e] + before + rank;
    }
    __syncthreads();
    if (leader && valid) {
      atomicAdd(&running[e], wcnt[wave * (E + 1) + e]);
      wcnt[wave * (E + 1) + e] = 0;
    }
    __syncthreads();
    if (in) {
      row_map[s] = row;
      if (valid) {
        row_src[row] = static_cast<int>(s) / K;   // slots < T * K < 2^31: 32-bit division
        row_k[row] = static_cast<int>(s) % K;
      }
      if (cache) slot_row[s - s0] = row;
    }
  }

  // 3. destinations for the reduce folded into the tiled GEMM2: the row of a
  // received row with exactly one local slot, whose expert has at least
  // min_tiled routes (the experts of the tiled kernel), names that slot;
  // other rows name none, and their received rows (and the ones with no
  // local slot) join tok_rest, in row order from this block's first entry.
  // This block's rows are its own received rows, so its row_map entries are
  // complete after the barrier; cnt[] holds the experts' totals.
  __syncthreads();
  for (int64_t tb = r0; tb < r1; tb += kThreads) {
    const int64_t t = tb + tid;
    bool rest = false;
    if (t < r1) {
      // this block's slots: from the LDS tables, or from row_map and idx if
      // too many (two separate loops, so that the LDS reads stay LDS reads
      // and do not become generic loads that wait for all memory)
      int n = 0, e1 = E;
      bool direct;
      if (cache) {
        const int* se = slot_e + (t * K - s0);
        const int* sr = slot_row + (t * K - s0);
#pragma unroll 8
        for (int k = 0; k < K; ++k) {
          if (sr[k] >= 0) {
            ++n;
            e1 = se[k];
          }
        }
        direct = n == 1 && cnt[e1] >= min_tiled;
#pragma unroll 8
        for (int k = 0; k < K; ++k) {
          const int m = sr[k];
          if (m >= 0) row_dst[m] = direct ? static_cast<int>(t * K + k) : -1;
        }
      } else {
        for (int k = 0; k < K; ++k) {
          const int64_t s = t * K + k;
          if (row_map[s] >= 0) {
            ++n;
            e1 = local_of(idx[s], eb, E);
          }
        }
        direct = n == 1 && cnt[e1] >= min_tiled;
        for (int k = 0; k < K; ++k) {
          const int m = row_map[t * K + k];
          if (m >= 0) row_dst[m] = direct ? static_cast<int>(t * K + k) : -1;
        }
      }
      rest = !direct;
    }
    const uint64_t mask = __ballot(rest);
    if (lane_id() == 0) tmp[wave] = __popcll(mask);
    __syncthreads();
    int before = 0, chunk = 0;
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) before += tmp[w];
      chunk += tmp[w];
    }
    if (rest) tok_rest[rest_at + before + popc_below(mask)] = static_cast<int>(t);
    rest_at += chunk;
    __syncthreads();
  }
}


// Small inputs (T * K <= kSmallSlots: decode batches): one block of kSlots
// threads (64, 256 or 1024, the fewest that hold every slot), one slot per
// thread and, for the row phase, one row per thread. Every global load (the
// slot's id, the rows' block counts) goes out at the start; the rest runs in
// LDS between block barriers:
//   0. the slot's local expert (E: none) into se[];
//   1. ranks among the wave's slots of the same expert (ids matched bit by
//      bit with ballots); each (wave, expert) leader stores its count;
//   2. per expert (a run of experts per thread): its count in each earlier
//      wave (an exclusive prefix over the waves), its total, and the segment
//      offsets (one block scan);
//   3. each local slot's row: offset + earlier waves' count + rank;
//   4. per received row: the fused GEMM2 destination of a row with exactly
//      one local slot of a tiled expert, and tok_rest in row order (a second
//      block scan).
// Same results, bit for bit, as the general kernels.
constexpr int kSmallSlots = 1024;

template <typename IdxT, int kSlots>
__global__ __launch_bounds__(kSlots) void route_small(
    const IdxT* __restrict__ idx, int T, int K, int64_t eb, int E, int B,
    const int* __restrict__ bc, int* __restrict__ counts, int* __restrict__ offsets,
    int* __restrict__ row_map, int* __restrict__ row_src, int* __restrict__ row_k,
    int* __restrict__ stats, int* __restrict__ row_dst, int* __restrict__ tok_rest,
    int min_tiled) {
  constexpr int kW = kSlots / kWave;
  constexpr int kPerE = kMaxE / kSlots;     // most experts per thread
  __shared__ int cw[kW * kMaxE];            // [wave][E] counts, then earlier waves' counts
  __shared__ int tot[kMaxE];                // routes per expert
  __shared__ int off[kMaxE];                // segment starts
  __shared__ int se[kSlots];                // slot's local expert (E: none)
  __shared__ int sr[kSlots];                // slot's expanded row (-1: none)
  __shared__ int tmp[kW];
  // [0] ignored slots, [1] rows with a local slot, [2] carrying rows,
  // [3] empty experts, [4] / [5] experts of the streaming / tiled GEMM
  __shared__ int misc[6];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int TK = T * K;                     // <= kSlots
  const int s = tid;                        // this thread's slot
  const int ts = s / K;                     // its received row

  // 0. the loads: the slot's id (clamped, so that it goes out at once) and,
  // for a padded plan, the block counts of the slot's row and of row tid;
  // a padding row's ids are never read
  IdxT id = 0;
  int bcs = 1, bct = 1;
  if (TK > 0) {
    if (B == 0) {
      id = idx[s < TK ? s : TK - 1];
    } else {
      bcs = bc[min(ts, T - 1) / B];
      bct = bc[min(tid, T - 1) / B];
    }
  }
  for (int i = tid; i < kW * E; i += kSlots) cw[i] = 0;
  if (tid < 6) misc[tid] = 0;
  const bool carry_s = s < TK && (B == 0 || ts - ts / B * B < bcs);
  if (B > 0 && carry_s) id = idx[s];
  const int e = carry_s ? local_of(id, eb, E) : E;
  const bool valid = e < E;
  se[s] = e;
  __syncthreads();

  // 1. rank among the wave's slots of the same expert
  const int nbits = 32 - __clz(E);          // bits of the values 0..E
  uint64_t peers = __ballot(1);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bal = __ballot(bit);
    peers &= bit ? bal : ~bal;
  }
  const int rank = popc_below(peers);
  if (valid && rank == 0) cw[wave * E + e] = __popcll(peers);
  const uint64_t ign = __ballot(carry_s && !valid);
  if (lane_id() == 0 && ign) atomicAdd(&misc[0], __popcll(ign));
  __syncthreads();

  // 2. per expert (experts tid * per .. + per - 1): earlier waves' counts,
  // totals, offsets
  const int per = (E + kSlots - 1) / kSlots;
  int te[kPerE];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kPerE; ++j) {
    te[j] = 0;
    const int x = tid * per + j;
    if (j < per && x < E) {
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        const int c = cw[w * E + x];
        cw[w * E + x] = te[j];
        te[j] += c;
      }
      sum += te[j];
    }
  }
  int R = 0;
  int o = block_exclusive_scan<kSlots>(sum, tmp, &R);
  int n_emp = 0, n_str = 0, n_til = 0;
#pragma unroll
  for (int j = 0; j < kPerE; ++j) {
    const int x = tid * per + j;
    if (j < per && x < E) {
      tot[x] = te[j];
      off[x] = o;
      counts[x] = te[j];
      offsets[x] = o;
      o += te[j];
      n_emp += te[j] == 0;
      n_str += te[j] > 0 && te[j] < min_tiled;
      n_til += te[j] >= min_tiled;
    }
  }
  if (tid == 0) offsets[E] = R;
  n_emp = wave_sum(n_emp);
  n_str = wave_sum(n_str);
  n_til = wave_sum(n_til);
  if (lane_id() == 0) {
    if (n_emp) atomicAdd(&misc[3], n_emp);
    if (n_str) atomicAdd(&misc[4], n_str);
    if (n_til) atomicAdd(&misc[5], n_til);
  }
  __syncthreads();

  // 3. the slot's row
  const int row = valid ? off[e] + cw[wave * E + e] + rank : -1;
  if (s < TK) {
    row_map[s] = row;
    if (valid) {
      row_src[row] = ts;
      row_k[row] = s - ts * K;
    }
  }
  sr[s] = row;
  __syncthreads();

  // 4. row tid: fused destination, tok_rest
  bool rest = false;
  int n = 0;
  if (tid < T) {
    int e1 = E;
    const int* re = se + tid * K;
    const int* rr = sr + tid * K;
    for (int k = 0; k < K; ++k) {
      if (rr[k] >= 0) {
        ++n;
        e1 = re[k];
      }
    }
    const bool direct = n == 1 && tot[e1] >= min_tiled;
    for (int k = 0; k < K; ++k) {
      const int m = rr[k];
      if (m >= 0) row_dst[m] = direct ? tid * K + k : -1;
    }
    rest = !direct;
  }
  const uint64_t loc = __ballot(n > 0);
  const uint64_t car = __ballot(tid < T && (B == 0 || tid - tid / B * B < bct));
  if (lane_id() == 0) {
    if (loc) atomicAdd(&misc[1], __popcll(loc));
    if (car) atomicAdd(&misc[2], __popcll(car));
  }
  int n_rest = 0;
  const int pos = block_exclusive_scan<kSlots>(rest ? 1 : 0, tmp, &n_rest);
  if (rest) tok_rest[pos] = tid;
  if (tid == 0) {
    stats[0] = R;
    stats[1] = misc[1];
    stats[2] = misc[0];
    stats[3] = misc[3];
    stats[4] = n_rest;
    stats[5] = misc[2];
    stats[6] = misc[4];
    stats[7] = misc[5];
  }
}

template <typename IdxT>
hipError_t launch(const tr_moe_plan& p, const IdxT* idx, hipStream_t st) {
  const tr_moe_desc& d = p.d;
  const int E = d.E, K = d.K;
  const int nb = p.scan_blocks, rpb = p.scan_rows_per_block;
  const size_t sh_scatter =
      sizeof(int) * (2 * E + kWaves * (E + 1) + hist_width(E) + kWaves + kMisc + 2 * kSlotCache);
  const int B = p.block_rows;
  const int* bc = p.block_counts;
  // fewest routes of an expert the grouped GEMM tiles (the others stream)
  const int min_tiled = min_tiled_routes(d);
  if (d.T * K <= kSmallSlots) {
    const int T = static_cast<int>(d.T), TK = T * K;
    if (TK <= 64)
      hipLaunchKernelGGL((route_small<IdxT, 64>), dim3(1), dim3(64), 0, st, idx, T, K,
                         d.expert_begin, E, B, bc, p.counts, p.offsets, p.row_map, p.row_src,
                         p.row_k, p.stats, p.row_dst, p.tok_rest, min_tiled);
    else if (TK <= 256)
      hipLaunchKernelGGL((route_small<IdxT, 256>), dim3(1), dim3(256), 0, st, idx, T, K,
                         d.expert_begin, E, B, bc, p.counts, p.offsets, p.row_map, p.row_src,
                         p.row_k, p.stats, p.row_dst, p.tok_rest, min_tiled);
    else
      hipLaunchKernelGGL((route_small<IdxT, kSmallSlots>), dim3(1), dim3(kSmallSlots), 0, st,
                         idx, T, K, d.expert_begin, E, B, bc, p.counts, p.offsets, p.row_map,
                         p.row_src, p.row_k, p.stats, p.row_dst, p.tok_rest, min_tiled);
    return hipGetLastError();
  }
  if (nb == 1) {
    hipLaunchKernelGGL((route_scatter<IdxT, true>), dim3(1), dim3(kThreads), sh_scatter, st, idx,
                       d.T, K, d.expert_begin, E, rpb, nb, B, bc, p.scan_tmp, p.counts, p.offsets,
                       p.row_map, p.row_src, p.row_k, p.stats, p.row_dst, p.tok_rest, min_tiled);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((route_count<IdxT>), dim3(nb), dim3(kThreads), sizeof(int) * hist_width(E),
                     st, idx, d.T, K, d.expert_begin, E, rpb, B, bc, p.scan_tmp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((route_scatter<IdxT, false>), dim3(nb), dim3(kThreads), sh_scatter, st, idx,
                     d.T, K, d.expert_begin, E, rpb, nb, B, bc, p.scan_tmp, p.counts, p.offsets,
                     p.row_map, p.row_src, p.row_k, p.stats, p.row_dst, p.tok_rest, min_tiled);
  return hipGetLastError();
}

}  // namespace

hipError_t route_scan(const tr_moe_plan& p, const void* idx, hipStream_t st) {
  if (p.d.idx_dtype == TR_IDX_I64) return launch(p, static_cast<const int64_t*>(idx), st);
  return launch(p, static_cast<const int32_t*>(idx), st);
}

void route_scan_geometry(int64_t T, int K, int* blocks, int* rows_per_block) {
  // One block for small inputs (up to kSmallSlots slots the single-block
  // kernel, up to 2048 the general one counting for itself: measured faster
  // than several blocks there, slower at 4096); otherwise ~512 slots per
  // block (two ranking rounds: the blocks are latency-bound, so more and
  // shorter ones), at most kMaxScanBlocks blocks.
  if (T * K <= 2048) {
    *blocks = 1;
    *rows_per_block = static_cast<int>(T > 0 ? T : 1);
    return;
  }
  int64_t rpb = cdiv(512, K);
  if (cdiv(T, rpb) > kMaxScanBlocks) rpb = cdiv(T, kMaxScanBlocks);
  *rows_per_block = static_cast<int>(rpb);
  *blocks = static_cast<int>(cdiv(T, rpb));
}

}  // namespace tr
