/*
 * Plain CPU oracle for one GPU's share of the expert-parallel MoE FFN.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library. It shares no code, header, table or
 * helper with the HIP library; neither includes or links the other.
 *
 * What it computes (DeepEP issue #48, "How to apply MoE MLP to recv_x ..."):
 * a rank receives each token once with its top-k expert ids; a grouped GEMM
 * needs every token copied once per local expert it is routed to ("expand"),
 * and a reduction folds the per-expert outputs back into one row per received
 * token before combine. Ids outside [expert_begin, expert_begin + E), -1
 * included, are not local and are skipped (DeepEP issue #760 repro: routes
 * below 0 are masked out before the local weight sum).
 *
 * Expert MLP: SwiGLU without bias. For expert e and input row x:
 *   g_i = sum_h W1[e][i][h] x_h,  u_i = sum_h W1[e][I+i][h] x_h   (i < I)
 *   h_i = silu(g_i) * u_i,        silu(z) = z / (1 + exp(-z))
 *   o_j = sum_i W2[e][j][i] h_i                                     (j < H)
 * Output row t: y_t = sum over local slots k, ascending, of w[t][k] * o.
 *
 * Floating point is double throughout, with no intermediate rounding. Inputs
 * are bf16 bit patterns (dtype 0) or float32 (dtype 1), widened exactly.
 *
 * Every function takes plain host pointers; all arrays are row-major.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Route table. idx [T*K]; outputs counts [E], offsets [E+1], row_map [T*K]
 * (expanded row or -1), row_src [R] (token), row_k [R] (slot). The caller
 * sizes row_src/row_k to at least T*K. Returns R. */
int64_t oracle_route(int64_t T, int32_t K, int64_t expert_begin, int32_t E,
                     const int64_t* idx, int32_t* counts, int32_t* offsets,
                     int32_t* row_map, int32_t* row_src, int32_t* row_k);

/* Route table of a padded buffer (SGLang PR #6092: DP workers' rows padded
 * to one size; padding rows hold no query). Rows form blocks of B rows; row t
 * carries a query when t - (t / B) B < block_counts[t / B], and the slots of
 * the other rows are not local whatever idx holds. B == 0: every row carries
 * (oracle_route). */
int64_t oracle_route_padded(int64_t T, int32_t K, int64_t expert_begin, int32_t E,
                            int32_t B, const int32_t* block_counts, const int64_t* idx,
                            int32_t* counts, int32_t* offsets, int32_t* row_map,
                            int32_t* row_src, int32_t* row_k);

/* Compaction of a padded buffer (SGLang PR #6092: only the effective rows go
 * to the communication buffer). The carrying rows (as in oracle_route_padded,
 * B >= 1), in row order, are compact rows 0, 1, ...; to_padded == 0 copies
 * each into its compact row of dst, to_padded == 1 copies compact row n of
 * src back to its padded row of dst (other dst rows untouched). Rows are
 * row_bytes bytes. Returns the number of carrying rows. */
int64_t oracle_compact_rows(int64_t T, int32_t B, const int32_t* block_counts,
                            int64_t row_bytes, const void* src, void* dst, int32_t to_padded);

/* Expand: Xe[r] = x[row_src[r]] for r < R, a bit copy of elem_bytes-wide
 * elements. */
void oracle_expand(int64_t R, int64_t H, int32_t elem_bytes, const void* x,
                   const int32_t* row_src, void* Xe);

/* One expert MLP on one input row, in double. w1e [2I*H], w2e [H*I], x [H]
 * (all of `dtype`); out [H]. */
void oracle_expert_mlp(int64_t H, int64_t I, int32_t dtype, const void* w1e,
                       const void* w2e, const void* x, double* out);

/* Expert outputs for a list of (expert, token) pairs: out [n, H] double.
 * experts[i] is a local expert index in [0, E). */
void oracle_expert_rows(int64_t n, const int32_t* experts, const int64_t* tokens,
                        int64_t H, int64_t I, int32_t dtype, const void* x,
                        const void* w1, const void* w2, double* out,
                        int32_t nthreads);

/* Weighted reduce: y[t] = sum over k ascending with row_map[t][k] >= 0 of
 * w[t][k] * O[row_map[t][k]] (w == NULL means weight 1). O is of `dtype`
 * (bf16 bits or float32), y [T, H] double. */
void oracle_combine(int64_t T, int32_t K, int64_t H, int32_t dtype,
                    const int32_t* row_map, const float* w, const void* O,
                    double* y);

/* Cross-rank combine epilogue (DeepEP issue #760, body: the epilogue sums,
 * for each output token, the rows returned by the ranks that hold its
 * experts; repro: combine without weights, so a token's result is the plain
 * sum of what it gets back). recv [N, H] of `dtype`; src [T, J]: src[t][j] is
 * the recv row of contribution j of token t, or -1 for none.
 *   y[t] = sum over j ascending with src[t][j] >= 0 of recv[src[t][j]]
 * y [T, H] double; a token with no contribution is 0. */
void oracle_combine_epilogue(int64_t T, int32_t J, int64_t H, int32_t dtype,
                             const int32_t* src, const void* recv, double* y);

/* Whole layer for the listed tokens (tokens == NULL: all T, in order).
 * y [n_tokens, H] double. Weights of non-local slots are never read. */
void oracle_forward(int64_t T, int32_t K, int64_t expert_begin, int32_t E,
                    int64_t H, int64_t I, int32_t dtype, const void* x,
                    const int64_t* idx, const float* w, const void* w1,
                    const void* w2, const int64_t* tokens, int64_t n_tokens,
                    double* y, int32_t nthreads);

/* silu in double, exposed so that its values can be pinned. */
double oracle_silu(double z);

/* Number of threads an oracle call with `nthreads` (<= 0: all) will use. */
int32_t oracle_threads(int32_t nthreads);

#ifdef __cplusplus
}
#endif
#endif
