// Internal launchers of libtopreduce (host side). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "topreduce.h"

namespace tr {

constexpr int kMaxScanBlocks = 256;
constexpr int kMaxK = 32;
constexpr int kMaxE = 1024;
// Experts with at most this many routes go to the weight-streaming GEMM.
constexpr int kStreamMaxRows = 32;
// A batch of at most this many expanded rows (T * K) sends every expert to the
// weight-streaming GEMM in the automatic mode: such experts rarely fill a
// tile, and the tiled kernels' launches would mostly find nothing to do.
constexpr int kSmallBatchRows = 128;
// The fewest routes of an expert the tiled GEMM takes under d's flags (the
// route scan marks the rows of such experts for the reduce folded into GEMM2).
inline int min_tiled_routes(const tr_moe_desc& d) {
  if (d.flags & TR_FLAG_GEMM_FORCE_STREAM) return 0x7fffffff;
  if (d.flags & TR_FLAG_GEMM_FORCE_TILED) return 1;
  return d.T * d.K <= kSmallBatchRows ? 0x7fffffff : kStreamMaxRows + 1;
}
// Spare rows after R_cap in the expanded (Xe) and intermediate (h) buffers,
// so GEMM tiles may read a full tile of rows from any segment start.
constexpr int kRowPad = 256;
// bf16 shapes of the tiled and streaming GEMM kernels: H a multiple of
// kColMultiple, I of kColMultiple / 2 (other shapes: the any-shape kernel).
constexpr int kColMultiple = 256;
// Most worker blocks of a DP-padded buffer (their counts' prefix sits in LDS).
constexpr int kMaxPadBlocks = 4096;

hipError_t route_scan(const tr_moe_plan& p, const void* idx, hipStream_t st);
void route_scan_geometry(int64_t T, int K, int* blocks, int* rows_per_block);
hipError_t expand(const tr_moe_plan& p, const void* x, hipStream_t st);
enum { kGemmUp = 1, kGemmDown = 2 };
// parts: kGemmUp (Xe -> h, SwiGLU), kGemmDown (h -> O), or both. With
// x_gather (bf16 only), GEMM1 reads the received rows x through the plan's
// route table instead of Xe, so no expand pass is needed.
// With y_fused (bf16 only), GEMM2 writes the rows of received rows with one
// local slot straight to y, weighted (w_fused, NULL for 1) and rounded as the
// reduce would; combine_reduce with skip_single then completes y. With
// y_done as well, a decode batch may run the whole reduce inside GEMM2: then
// *y_done is set and y is complete (no combine_reduce needed).
hipError_t grouped_gemm(const tr_moe_plan& p, const void* w1, const void* w2, int parts,
                        hipStream_t st, const void* x_gather = nullptr,
                        const float* w_fused = nullptr, void* y_fused = nullptr,
                        bool* y_done = nullptr);
// Whether GEMM1 may gather from x of this shape (32-bit buffer offsets).
bool gemm_can_gather(const tr_moe_desc& d);
hipError_t combine_reduce(const tr_moe_plan& p, const void* expert_out, const float* w, void* y,
                          hipStream_t st, bool skip_single = false);
// y[t] = sum over j of recv[src[t][j]] (src >= 0 and < n_recv), unit weights.
hipError_t combine_epilogue(int64_t T, int J, int64_t H, bool bf16, const int* src,
                            const void* recv, int64_t n_recv, void* y, hipStream_t st);

// Rows of a DP-padded buffer that carry data (block j of B rows: its first
// counts[j], clamped) copied to compact order, or back (to_padded).
hipError_t compact_rows(int64_t T, int B, const int* counts, int64_t row_bytes, const void* src,
                        void* dst, bool to_padded, int* n_out, hipStream_t st);

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace tr
