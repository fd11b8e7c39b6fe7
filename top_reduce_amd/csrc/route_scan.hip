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
//  - a small input (T*K <= 4096) runs as one block that counts for itself:
//    one launch instead of two.
//  - a DP-padded buffer (SGLang PR #6092: workers' batches padded to one
//    shape) names per block of rows how many carry tokens; the other rows are
//    treated as rows without a local slot, and their ids are never loaded.
#include "tr_device.h"
#include "tr_internal.h"

namespace tr {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

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
  const int64_t j = r / B;
  return r - j * B < bc[j];
}

// Adds the slots of rows [r0, r1) to cnt[0..E+3): per-expert counts, then
// cnt[E] = ignored slots, cnt[E+1] = rows with at least one local slot,
// cnt[E+2] = rows that carry a token. Rows that do not carry one count in
// none of them.
template <typename IdxT>
__device__ void count_rows(const IdxT* __restrict__ idx, int64_t r0, int64_t r1, int K,
                           int64_t eb, int E, int B, const int* __restrict__ bc, int* cnt) {
  const int64_t s0 = r0 * K, s1 = r1 * K;
  for (int64_t base = s0; base < s1; base += kThreads) {
    const int64_t s = base + threadIdx.x;
    const bool in = s < s1 && (B == 0 || carries(s / K, B, bc));
    const int e = in ? local_of(idx[s], eb, E) : E;
    if (e < E) atomicAdd(&cnt[e], 1);
    const uint64_t ign = __ballot(in && e == E);
    if (lane_id() == 0 && ign) atomicAdd(&cnt[E], __popcll(ign));
  }
  for (int64_t base = r0; base < r1; base += kThreads) {
    const int64_t r = base + threadIdx.x;
    const bool in = r < r1 && (B == 0 || carries(r, B, bc));
    bool any = false;
    if (in)
      for (int k = 0; k < K; ++k) any |= local_of(idx[r * K + k], eb, E) < E;
    const uint64_t m = __ballot(any);
    if (lane_id() == 0 && m) atomicAdd(&cnt[E + 1], __popcll(m));
    const uint64_t c = __ballot(in);
    if (lane_id() == 0 && c) atomicAdd(&cnt[E + 2], __popcll(c));
  }
}

template <typename IdxT>
__global__ __launch_bounds__(kThreads) void route_count(const IdxT* __restrict__ idx, int64_t T,
                                                        int K, int64_t eb, int E, int rpb, int B,
                                                        const int* __restrict__ bc,
                                                        int* __restrict__ hist,
                                                        int* __restrict__ stats) {
  extern __shared__ int cnt[];
  if (blockIdx.x == 0 && threadIdx.x == 0) stats[4] = 0;   // tok_rest entries (route_scatter)
  for (int i = threadIdx.x; i < E + 3; i += kThreads) cnt[i] = 0;
  __syncthreads();
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rpb;
  const int64_t r1 = r0 + rpb < T ? r0 + rpb : T;
  count_rows(idx, r0, r1, K, eb, E, B, bc, cnt);
  __syncthreads();
  for (int i = threadIdx.x; i < E + 3; i += kThreads) hist[blockIdx.x * (E + 3) + i] = cnt[i];
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
  int* base = sh;                       // [E] first row of this block's slots per expert
  int* running = base + E;              // [E] rows taken so far by this block
  int* wcnt = running + E;              // [kWaves][E + 1] per-wave counts of a round
  int* cnt = wcnt + kWaves * (E + 1);   // [E + 3] own counts (kSelf)
  int* tmp = cnt + (E + 3);             // [kWaves] scan scratch
  int* misc = tmp + kWaves;             // [4]

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rpb;
  const int64_t r1 = r0 + rpb < T ? r0 + rpb : T;

  int* prior = wcnt;                    // [E] phase 1 only; wcnt is zeroed after
  for (int i = tid; i < E + 3; i += kThreads) cnt[i] = 0;
  for (int i = tid; i < E; i += kThreads) prior[i] = 0;
  if (tid < 4) misc[tid] = 0;
  if (kSelf && tid == 0) stats[4] = 0;   // tok_rest entries (phase 3)
  __syncthreads();
  if (kSelf) {
    count_rows(idx, r0, r1, K, eb, E, B, bc, cnt);
  } else {
    // totals and this block's prior counts from every block's partials; all
    // threads share the (block, expert) grid so the loads are independent
    const int n = nblocks * E;
    for (int i = tid; i < n; i += kThreads) {
      const int b = i / E, e = i - b * E;
      const int c = hist[b * (E + 3) + e];
      if (c) {
        atomicAdd(&cnt[e], c);
        if (b < static_cast<int>(blockIdx.x)) atomicAdd(&prior[e], c);
      }
    }
  }
  __syncthreads();

  // 1. totals per expert, this block's prior count, segment offsets.
  const int per = (E + kThreads - 1) / kThreads;  // experts per thread (<= 4)
  int tsum = 0;
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
    }
  }
  __syncthreads();                      // prior[] read; wcnt becomes per-wave counts
  for (int i = tid; i < kWaves * (E + 1); i += kThreads) wcnt[i] = 0;
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
      }
      off += tot[j];
    }
  }
  if (blockIdx.x == 0) {
    // ignored slots, rows with a local route and carrying rows, summed
    // over blocks
    if (kSelf) {
      if (tid == 0) { misc[1] = cnt[E]; misc[2] = cnt[E + 1]; misc[3] = cnt[E + 2]; }
    } else {
      int ign = 0, tl = 0, cr = 0;
      for (int b = tid; b < nblocks; b += kThreads) {
        ign += hist[b * (E + 3) + E];
        tl += hist[b * (E + 3) + E + 1];
        cr += hist[b * (E + 3) + E + 2];
      }
      if (ign) atomicAdd(&misc[1], ign);
      if (tl) atomicAdd(&misc[2], tl);
      if (cr) atomicAdd(&misc[3], cr);
    }
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid == 0) {
    offsets[E] = R;
    stats[0] = R;
    stats[1] = misc[2];
    stats[2] = misc[1];
    stats[3] = misc[0];
    stats[5] = misc[3];
  }

  // 2. stable ranks, one round of kThreads slots at a time.
  const int nbits = 32 - __clz(E);  // bits of the values 0..E
  const int64_t s0 = r0 * K, s1 = r1 * K;
  for (int64_t rb = s0; rb < s1; rb += kThreads) {
    const int64_t s = rb + tid;
    const bool in = s < s1;
    const int e = in && (B == 0 || carries(s / K, B, bc)) ? local_of(idx[s], eb, E) : E;
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
        row_src[row] = static_cast<int>(s / K);
        row_k[row] = static_cast<int>(s % K);
      }
    }
  }

  // 3. destinations for the reduce folded into the tiled GEMM2: the row of a
  // received row with exactly one local slot, whose expert has at least
  // min_tiled routes (the experts of the tiled kernel), names that slot;
  // other rows name none, and their received rows (and the ones with no
  // local slot) join tok_rest. This block's rows are its own received rows,
  // so its row_map entries are complete after the barrier; cnt[] holds the
  // experts' totals.
  __syncthreads();
  for (int64_t tb = r0; tb < r1; tb += kThreads) {
    const int64_t t = tb + tid;
    bool rest = false;
    if (t < r1) {
      int n = 0, k1 = 0;
      for (int k = 0; k < K; ++k)
        if (row_map[t * K + k] >= 0) {
          ++n;
          k1 = k;
        }
      const bool direct = n == 1 && cnt[local_of(idx[t * K + k1], eb, E)] >= min_tiled;
      for (int k = 0; k < K; ++k) {
        const int m = row_map[t * K + k];
        if (m >= 0) row_dst[m] = direct ? static_cast<int>(t * K + k) : -1;
      }
      rest = !direct;
    }
    const uint64_t mask = __ballot(rest);
    int at = 0;
    if (lane_id() == 0 && mask) at = atomicAdd(&stats[4], __popcll(mask));
    at = __shfl(at, 0);
    if (rest) tok_rest[at + popc_below(mask)] = static_cast<int>(t);
  }
}

template <typename IdxT>
hipError_t launch(const tr_moe_plan& p, const IdxT* idx, hipStream_t st) {
  const tr_moe_desc& d = p.d;
  const int E = d.E, K = d.K;
  const int nb = p.scan_blocks, rpb = p.scan_rows_per_block;
  const size_t sh_scatter = sizeof(int) * (2 * E + kWaves * (E + 1) + (E + 3) + kWaves + 4);
  const int B = p.block_rows;
  const int* bc = p.block_counts;
  // fewest routes of an expert the grouped GEMM tiles (the others stream)
  const int min_tiled = (d.flags & TR_FLAG_GEMM_FORCE_STREAM) ? INT32_MAX
                        : (d.flags & TR_FLAG_GEMM_FORCE_TILED) ? 1 : kStreamMaxRows + 1;
  if (nb == 1) {
    // one block: its route_scatter zeroes the tok_rest count itself
    hipLaunchKernelGGL((route_scatter<IdxT, true>), dim3(1), dim3(kThreads), sh_scatter, st, idx,
                       d.T, K, d.expert_begin, E, rpb, nb, B, bc, p.scan_tmp, p.counts, p.offsets,
                       p.row_map, p.row_src, p.row_k, p.stats, p.row_dst, p.tok_rest, min_tiled);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((route_count<IdxT>), dim3(nb), dim3(kThreads), sizeof(int) * (E + 3), st,
                     idx, d.T, K, d.expert_begin, E, rpb, B, bc, p.scan_tmp, p.stats);
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
  // One block for small inputs; otherwise ~1024 slots per block, at most
  // kMaxScanBlocks blocks.
  if (T * K <= 4096) {
    *blocks = 1;
    *rows_per_block = static_cast<int>(T > 0 ? T : 1);
    return;
  }
  int64_t rpb = cdiv(1024, K);
  if (cdiv(T, rpb) > kMaxScanBlocks) rpb = cdiv(T, kMaxScanBlocks);
  *rows_per_block = static_cast<int>(rpb);
  *blocks = static_cast<int>(cdiv(T, rpb));
}

}  // namespace tr
