/*
 * topreduce.h -- C ABI of libtopreduce.so: one GPU's share of an
 * expert-parallel MoE FFN on MI355X (gfx950).
 *
 * The problem (DeepEP issue #48, "How to apply MoE MLP to recv_x returned by
 * dispatch when num_expert_per_rank > 1", question and answers): after
 * dispatch a rank holds each received token once, as a row of recv_x, with its
 * top-k expert ids and gate weights. To run the local experts as a grouped
 * GEMM every token is expanded once per local expert it is routed to; after
 * the experts, a reduction folds each token's expert outputs back into one row
 * so that the result keeps recv_x's row count and order, which combine's
 * dispatch handle requires. DeepEP issue #760 ("DeepEP V2 combine epilogue low
 * batch performance") shows this weighted reduce as the combine epilogue and
 * its low-batch straggling when one warp serves one token.
 *
 * The path, per call sequence:
 *   moe_plan     route scan: per-expert counts and segment offsets, and the
 *                stable maps between received slots and expanded rows
 *   moe_plan_padded  the same over a DP-padded buffer whose padding rows
 *                carry no query; moe_compact_rows copies only the effective
 *                rows of such a buffer, and back
 *   moe_forward  = moe_expand + moe_grouped_gemm + moe_combine_reduce; bf16
 *                runs the fused forms moe_grouped_gemm_up_x (GEMM1 straight
 *                from x), moe_grouped_gemm_down_y (GEMM2 writing rows with one
 *                local slot straight to y) and moe_combine_reduce_multi, fp32
 *                moe_grouped_gemm_up_x, with the same result bit for bit
 *
 * Conventions for every entry point:
 *  - Pointers named "device" are HIP device (or managed) memory; the others
 *    are host memory. The caller allocates and owns every buffer, including
 *    the workspace; the library allocates nothing and keeps no per-call state
 *    (moe_forward_noalloc alone works in a workspace the library holds as a
 *    static device array).
 *  - All work is enqueued on `stream` (NULL: the null stream) and returns
 *    without synchronising, except moe_plan_stats, which waits on `stream`.
 *    Calls are graph-capturable except moe_plan_stats.
 *  - Arrays are dense and row-major. x, y, W1, W2 and the expert buffers are
 *    all of one element type, desc->dtype.
 *  - Shapes: H a multiple of 8 (rows of x, y and the expert buffers move in
 *    16-byte pieces), any I; other H return TR_EUNSUPPORTED. bf16 shapes with
 *    H a multiple of 256 and I a multiple of 128 run the tiled / streaming
 *    GEMM kernels; the others run one any-shape kernel for both GEMMs (32 x 32
 *    tiles per wave, operands from L2; the GEMM force flags then only change
 *    which rows the reduce folded into GEMM2 takes).
 *  - Errors: a non-zero tr_status and a message in moe_last_error(). Argument
 *    checks happen on the host before anything is enqueued. Nothing aborts.
 *  - Ids outside [expert_begin, expert_begin + E), -1 included, are routes to
 *    other ranks or padding: they are ignored, never an error, and their
 *    weights are never read (DeepEP issue #760, repro script: routes below 0
 *    are masked out before the local weight sum).
 */
#ifndef TOPREDUCE_H
#define TOPREDUCE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TR_ABI_VERSION 5

typedef enum {
    TR_OK = 0,
    TR_EINVAL = -1,        /* bad argument: null/misaligned pointer, bad size */
    TR_EUNSUPPORTED = -2,  /* valid but not supported shape or dtype */
    TR_EWORKSPACE = -3,    /* workspace smaller than moe_workspace_size() */
    TR_EHIP = -4           /* a HIP runtime call failed */
} tr_status;

typedef enum { TR_BF16 = 0, TR_F32 = 1 } tr_dtype;
typedef enum { TR_IDX_I32 = 0, TR_IDX_I64 = 1 } tr_idx_dtype;

/* Grouped-GEMM kernel choice. AUTO sends experts with at most 32 routes to the
 * weight-streaming kernel and the others to the tiled MFMA kernel, and every
 * expert to the weight-streaming kernel when T * K <= 128; the FORCE flags
 * send every expert to one of them (for testing). */
#define TR_FLAG_GEMM_FORCE_TILED 0x1
#define TR_FLAG_GEMM_FORCE_STREAM 0x2
/* No expanded-row buffer: the workspace holds no Xe (it shrinks by
 * (T * K + 256) * H * 2 bytes) and the plan's Xe is NULL. Only the forms that
 * gather from x work: moe_forward, moe_grouped_gemm_up_x and the entry points
 * that do not touch Xe. moe_expand, moe_grouped_gemm and moe_grouped_gemm_up
 * return TR_EUNSUPPORTED. Needs bf16 and T * H * 2 < 2^31, else the
 * descriptor is TR_EUNSUPPORTED. */
#define TR_FLAG_NO_XE 0x4

typedef struct tr_moe_desc {
    int64_t T;             /* received rows (recv_x rows), >= 0 */
    int32_t K;             /* top-k slots per row, 1..32 */
    int32_t E;             /* local experts, 1..1024 */
    int64_t expert_begin;  /* global id of local expert 0 */
    int64_t H;             /* hidden size */
    int64_t I;             /* SwiGLU intermediate size */
    int32_t dtype;         /* tr_dtype of x, y, W1, W2 */
    int32_t idx_dtype;     /* tr_idx_dtype of topk_idx */
    int32_t flags;         /* TR_FLAG_* */
    int32_t reserved;
} tr_moe_desc;

/* Host-side handle returned by moe_plan: the descriptor plus device pointers
 * into the caller's workspace. Valid while that workspace lives and until the
 * next moe_plan on the same workspace; reusable for any number of forwards.
 * Row-index arrays are int32. */
typedef struct tr_moe_plan {
    tr_moe_desc d;
    int64_t R_cap;         /* T * K: upper bound of expanded rows */
    void* ws;
    size_t ws_bytes;
    int32_t* counts;       /* [E] routes per local expert */
    int32_t* offsets;      /* [E+1] segment starts; offsets[E] = R */
    int32_t* row_map;      /* [T*K] expanded row of slot (t,k), or -1 */
    int32_t* row_src;      /* [R_cap] received row of expanded row r (r < R) */
    int32_t* row_k;        /* [R_cap] slot of expanded row r (r < R) */
    int32_t* stats;        /* [8] R, rows with >= 1 local route, ignored slots, empty
                              experts, entries of tok_rest, rows that carry a
                              token (T, or the carrying rows of a padded plan),
                              non-empty experts the streaming GEMM takes (fewer
                              than 33 routes, any number when T * K <= 128;
                              every one with TR_FLAG_GEMM_FORCE_STREAM, none
                              with TR_FLAG_GEMM_FORCE_TILED), non-empty experts
                              the tiled GEMM takes (the others) */
    int32_t* scan_tmp;     /* route-scan block partials */
    void* Xe;              /* [R_cap + 256, H] expanded rows (expert-contiguous);
                              NULL with TR_FLAG_NO_XE */
    void* h;               /* [R_cap + 256, I] silu(gate) * up */
    void* O;               /* [R_cap, H] expert outputs */
    int32_t scan_blocks;
    int32_t scan_rows_per_block;
    int32_t* row_dst;      /* [R_cap] for expanded row r < R: slot t*K + k if its
                              received row t has exactly one local slot and its
                              expert is one the tiled GEMM takes (see
                              moe_grouped_gemm_down_y), else -1 */
    int32_t* tok_rest;     /* [T] the other received rows, in ascending order;
                              stats[4] of them */
    int32_t block_rows;    /* moe_plan_padded: rows per worker block; 0 otherwise */
    int32_t reserved2;
    const int32_t* block_counts;  /* moe_plan_padded: the caller's block_counts */
} tr_moe_plan;

/* Bytes of device workspace a plan for `desc` needs (every buffer above,
 * 256-byte aligned). Returns 0 and sets the last error if desc is invalid. */
size_t moe_workspace_size(const tr_moe_desc* desc);

/* Route scan (DeepEP issue #48 answer: expand each token to its experts before
 * the grouped GEMM). topk_idx: device [T, K] of idx_dtype, global expert ids
 * or -1. ws: device, ws_bytes >= moe_workspace_size(desc), 256-byte aligned.
 * Fills *out (host) and enqueues the scan: counts, offsets, row_map, row_src,
 * row_k and stats are written on the device. Row order: an expert's segment
 * lists its routes by received row, then by slot. Bit-exact and deterministic.
 * topk_idx may be freed once the stream has passed this call. */
tr_status moe_plan(const tr_moe_desc* desc, const void* topk_idx, void* ws, size_t ws_bytes,
                   hipStream_t stream, tr_moe_plan* out);

/* Route scan of a DP-padded received buffer (SGLang PR #6092: data-parallel
 * workers of different batch sizes share one FFN input of fixed shape, each
 * worker's rows padded to the largest batch; padded rows hold no query and
 * must cost no expert work). The T rows are split into blocks of block_rows
 * rows (the last block may be shorter), one per worker; the first
 * block_counts[j] rows of block j carry tokens and the rest are padding.
 * Padding rows are rows without a local slot whatever topk_idx holds there
 * (their ids are never read): they get no expanded row and no GEMM work,
 * their row_map entries are -1, they count in none of stats[0..2], and the
 * forward writes them as +0. Otherwise exactly moe_plan, which is this call
 * with every row carrying. block_counts: device int32
 * [ceil(T / block_rows)], each value clamped to [0, rows of the block]; read by the
 * scan only (it may change after the stream has passed this call, but then
 * moe_compact_rows must be given the same counts). block_rows >= 1 and at
 * most 4096 blocks, else TR_EUNSUPPORTED. */
tr_status moe_plan_padded(const tr_moe_desc* desc, const void* topk_idx, int32_t block_rows,
                          const int32_t* block_counts, void* ws, size_t ws_bytes,
                          hipStream_t stream, tr_moe_plan* out);

/* Compaction of a DP-padded buffer (SGLang PR #6092, answer: only each
 * worker's effective rows are copied into the communication buffer, never the
 * padding). Rows are row_bytes bytes; the T padded rows form blocks of
 * block_rows rows whose first block_counts[j] rows (clamped to
 * [0, block_rows]) carry data, and the compact order is block by block, row
 * order inside a block. to_padded == 0: compact row i = the i-th carrying
 * padded row, for every carrying row (padded -> compact, as before the
 * all-gather). to_padded == 1: the reverse, carrying padded row = its compact
 * row; padding rows are left untouched (compact -> padded, handing each
 * worker its rows back). n_out: device int32 or NULL; receives the number of
 * carrying rows. src: device [T or compact rows, row_bytes]; dst likewise;
 * no overlap. row_bytes a positive multiple of 4 with src and dst 4-byte
 * aligned (16-byte copies when row_bytes and both pointers allow); at most
 * 4096 blocks and T < 2^31 (else TR_EUNSUPPORTED); T == 0 writes only n_out.
 * Bit copies: works for x, topk_idx
 * and topk_weights alike. */
tr_status moe_compact_rows(int64_t T, int32_t block_rows, const int32_t* block_counts,
                           int64_t row_bytes, const void* src, void* dst, int32_t to_padded,
                           int32_t* n_out, hipStream_t stream);

/* Whole layer: y[t] = sum over local slots k (ascending) of
 * topk_weights[t][k] * MLP_e(x[t]), with MLP_e(x) = W2[e] (silu(W1[e][0:I] x) *
 * (W1[e][I:2I] x)). Rows without a local slot are written as +0.
 * x: device [T, H]; topk_weights: device fp32 [T, K] or NULL for weight 1
 * (combine called without weights in DeepEP issue #760's repro);
 * w1: device [E, 2I, H] (rows [0, I) gate, [I, 2I) up); w2: device [E, H, I];
 * y: device [T, H], may alias x; no other aliasing. Accumulation is fp32;
 * for bf16 the intermediate h and expert outputs are rounded to bf16.
 * y equals, bit for bit, moe_expand, moe_grouped_gemm and
 * moe_combine_reduce(plan, NULL, topk_weights, y). For bf16 with
 * T * H * 2 < 2^31 it runs moe_grouped_gemm_up_x, moe_grouped_gemm_down_y and
 * moe_combine_reduce_multi instead (the fused forms of expand and of the
 * reduce): Xe is not written, and O only for received rows with several
 * local slots. With enough tiles for several rounds the two GEMMs run as
 * three launches (GEMM1's whole rounds; its last round beside GEMM2 tiles of
 * rows GEMM1 has finished; the rest of GEMM2), with the same result. A
 * decode batch (at most 32 expanded rows, automatic GEMM mode) runs the
 * reduce inside GEMM2's launch, again with the same result, and writes no O
 * (DeepEP issue #760, body: the separate low-batch epilogue left out). */
tr_status moe_forward(const tr_moe_plan* plan, const void* x, const float* topk_weights,
                      const void* w1, const void* w2, void* y, hipStream_t stream);

/* Expand (DeepEP issue #48 answer): Xe[r] = x[row_src[r]] for r < R, a bit
 * copy into the plan's expert-contiguous buffer. x: device [T, H]. */
tr_status moe_expand(const tr_moe_plan* plan, const void* x, hipStream_t stream);

/* Grouped SwiGLU GEMM over the plan's Xe: h = silu(Xe W1g^T) * (Xe W1u^T) per
 * expert segment, then O = h W2^T. Empty experts and rows past each segment
 * cost no MFMA work (SGLang PR #6092: padded rows must not add computation). */
tr_status moe_grouped_gemm(const tr_moe_plan* plan, const void* w1, const void* w2,
                           hipStream_t stream);

/* The two halves of moe_grouped_gemm, for callers that fuse or time them
 * separately: _up computes h from the plan's Xe and w1 (GEMM1 with the SwiGLU
 * epilogue), _down computes O from h and w2. Running _up then _down on one
 * stream is exactly moe_grouped_gemm. */
tr_status moe_grouped_gemm_up(const tr_moe_plan* plan, const void* w1, hipStream_t stream);
/* GEMM1 with the SwiGLU epilogue straight from the received rows: the
 * activation tiles are gathered from x (device [T, H]) through the plan's route
 * table, so no expand pass and no Xe are needed (the fused form of the
 * expand step). h equals moe_expand followed by moe_grouped_gemm_up. fp32, and
 * bf16 with T * H * 2 < 2^31; otherwise (bf16 with a larger x) it runs
 * moe_expand and moe_grouped_gemm_up. */
tr_status moe_grouped_gemm_up_x(const tr_moe_plan* plan, const void* x, const void* w1,
                                hipStream_t stream);
tr_status moe_grouped_gemm_down(const tr_moe_plan* plan, const void* w2, hipStream_t stream);
/* GEMM2 with the weighted reduce folded into its epilogue for received rows
 * with exactly one local slot whose expert the tiled kernel takes (more than
 * 32 routes in a batch of T * K > 128; every expert with
 * TR_FLAG_GEMM_FORCE_TILED, none with TR_FLAG_GEMM_FORCE_STREAM): the plan's
 * row_dst. Such a row's output is
 * rounded to bf16 as O would be, weighted and rounded again exactly as
 * moe_combine_reduce does, and written straight to y[t]; the other rows go to
 * O. topk_weights: device fp32 [T, K] or NULL (weight 1); y: device [T, H],
 * must not overlap h or O. moe_combine_reduce_multi then completes y. bf16 with
 * T * H * 2 < 2^31 only; otherwise TR_EUNSUPPORTED (use moe_grouped_gemm_down
 * and moe_combine_reduce). */
tr_status moe_grouped_gemm_down_y(const tr_moe_plan* plan, const void* w2,
                                  const float* topk_weights, void* y, hipStream_t stream);

/* Weighted top-k reduce (DeepEP issue #48: the reduction before the combine
 * all-to-all; DeepEP issue #760: the combine epilogue, one row per received
 * token): y[t] = sum over k ascending with row_map[t][k] >= 0 of
 * topk_weights[t][k] * expert_out[row_map[t][k]], accumulated in fp32.
 * expert_out: device [>= R, H] of dtype, or NULL for the plan's O.
 * topk_weights: device fp32 [T, K] or NULL (weight 1). y: device [T, H].
 * The hidden dimension is split across wavefronts so that a few tokens still
 * occupy many compute units. */
tr_status moe_combine_reduce(const tr_moe_plan* plan, const void* expert_out,
                             const float* topk_weights, void* y, hipStream_t stream);

/* moe_combine_reduce over the plan's O for the received rows in the plan's
 * tok_rest only; the others are left as moe_grouped_gemm_down_y wrote them. */
tr_status moe_combine_reduce_multi(const tr_moe_plan* plan, const float* topk_weights, void* y,
                                   hipStream_t stream);

/* Cross-rank combine epilogue (DeepEP issue #760, body: after combine's
 * all-to-all, every output token sums the rows returned by the ranks that
 * hold its experts; the repro's combine takes no weights). Standalone: no
 * plan.
 *   y[t] = sum over j ascending with 0 <= src[t][j] < n_recv of recv[src[t][j]]
 * accumulated in fp32 and rounded once to dtype; a token with no
 * contribution is +0. recv: device [n_recv, H] rows of dtype (e.g. the P
 * ranks' partial rows one after the other); src: device int32 [T, J], -1 for
 * no contribution (indices >= n_recv count as none); y: device [T, H], must
 * not overlap recv. The hidden dimension is split across wavefronts (512
 * elements each), so a handful of tokens still occupies many compute units.
 * Shapes: 1 <= J <= 65536, H a multiple of 8; T == 0 is a no-op. recv and y
 * 16-byte aligned, src 4-byte aligned. */
tr_status moe_combine_epilogue(int64_t T, int32_t J, int64_t H, tr_dtype dtype,
                               const int32_t* src, const void* recv, int64_t n_recv, void* y,
                               hipStream_t stream);

/* Bytes of the library's own static workspace on each device, used by
 * moe_forward_noalloc only. */
#define TR_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. moe_plan
 * followed by moe_forward, with the workspace taken from a device array the
 * library holds (TR_NOALLOC_SCRATCH_BYTES per device, from module load until
 * the process ends) instead of the caller's. The result equals moe_plan +
 * moe_forward bit for bit. Calls no hipMalloc, hipFree or allocating library
 * routine.
 *   desc, topk_idx: as moe_plan; x, topk_weights, w1, w2, y: as moe_forward.
 *   bf16 plans without the expanded-row buffer (TR_FLAG_NO_XE is added when
 *   allowed), so the batch fits when moe_workspace_size of that descriptor is
 *   at most TR_NOALLOC_SCRATCH_BYTES (decode and small prefill batches, e.g.
 *   T = 64, K = 16, H = 3584, I = 2048 needs about 13 MB); larger batches
 *   return TR_EUNSUPPORTED before anything is enqueued.
 * Every call on one device shares that device's array and leaves its last
 * contents there (nothing in it needs to start zeroed: the route scan writes
 * every entry the later kernels read). Calls that overlap on one device (two
 * streams, or two threads, without ordering between them) race on it. */
tr_status moe_forward_noalloc(const tr_moe_desc* desc, const void* topk_idx, const void* x,
                              const float* topk_weights, const void* w1, const void* w2,
                              void* y, hipStream_t stream);

/* Copies stats to host_out[4] = {R, rows with a local route, ignored slots,
 * empty experts} and synchronises `stream` (opt-in host sync, the counterpart
 * of dispatch's do_cpu_sync in DeepEP issue #760's repro). */
tr_status moe_plan_stats(const tr_moe_plan* plan, int32_t* host_out, hipStream_t stream);

/* Message of the last error on the calling thread ("" if none). */
const char* moe_last_error(void);

/* TR_ABI_VERSION of the built library. */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
