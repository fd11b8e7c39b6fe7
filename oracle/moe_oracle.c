/*
 * Plain CPU oracle for one GPU's share of the expert-parallel MoE FFN.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * bench's CPU-baseline leg, never by the library it checks. Every step below
 * is the definition written out as loops, in double, with no blocking or
 * reordering beyond the definition. Threads (OpenMP) only split independent
 * tokens or rows.
 *
 * Sources (page titles; sections):
 *  - DeepEP issue #48, "How to apply MoE MLP to recv_x returned by dispatch
 *    when num_expert_per_rank > 1": the question (a token is received once
 *    with its top-k ids; duplicating it per expert breaks combine's handle, so
 *    the output keeps recv_x's row count) and the answers (expand each token to
 *    its experts for the grouped GEMM; a reduction before the combine
 *    all-to-all folds them back).
 *  - DeepEP issue #760, "DeepEP V2 combine epilogue low batch performance":
 *    the repro script (routes with id < 0 are masked out; padding rows carry
 *    all -1 routes and zero weights; combine without weights is a plain sum).
 *  - The expert MLP form is a reading: the pages say only "group gemm based
 *    MLP"; it is taken as SwiGLU with W1's first I rows the gate, no bias.
 *  - SGLang PR #6092, review thread: data-parallel workers of unequal batch
 *    sizes share one FFN input buffer, each worker's rows padded to a common
 *    size; padded rows hold no query (sequence length 0) and cost no
 *    computation, and only each worker's effective rows are copied into the
 *    communication buffer.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the top half of an IEEE float32: widening is a 16-bit shift. */
static double widen_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double elem(const void* p, int32_t dtype, int64_t i) {
    if (dtype == 0) return widen_bf16(((const uint16_t*)p)[i]);
    return (double)((const float*)p)[i];
}

static int64_t elem_bytes(int32_t dtype) { return dtype == 0 ? 2 : 4; }

int32_t oracle_threads(int32_t nthreads) {
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* A slot is local when its id lies in this rank's expert range. */
static int local_expert(int64_t id, int64_t expert_begin, int32_t E) {
    int64_t e = id - expert_begin;
    return (e >= 0 && e < (int64_t)E) ? (int)e : -1;
}

/* Rows of a padded buffer: block j = t / B holds rows [j B, j B + B); its
 * first block_counts[j] rows carry a query. B == 0: no padding, every row
 * carries. */
static int carries_row(int64_t t, int32_t B, const int32_t* block_counts) {
    if (B == 0) return 1;
    int64_t j = t / B;
    return t - j * B < (int64_t)block_counts[j];
}

/* Local expert of slot (t, k), or -1; a padding row has no local slot. */
static int slot_expert(int64_t t, int32_t k, int32_t K, int64_t expert_begin, int32_t E,
                       const int64_t* idx, int32_t B, const int32_t* block_counts) {
    if (!carries_row(t, B, block_counts)) return -1;
    return local_expert(idx[t * K + k], expert_begin, E);
}

int64_t oracle_route_padded(int64_t T, int32_t K, int64_t expert_begin, int32_t E,
                            int32_t B, const int32_t* block_counts, const int64_t* idx,
                            int32_t* counts, int32_t* offsets, int32_t* row_map,
                            int32_t* row_src, int32_t* row_k) {
    /* 1. per-expert route counts */
    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t t = 0; t < T; ++t)
        for (int32_t k = 0; k < K; ++k) {
            int e = slot_expert(t, k, K, expert_begin, E, idx, B, block_counts);
            if (e >= 0) counts[e] += 1;
        }
    /* 2. segment starts: exclusive prefix sum; offsets[E] = R */
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    /* 3. walk the slots token-major, slot-minor; the j-th local route to
     *    expert e takes row offsets[e] + j */
    int32_t* fill = (int32_t*)calloc((size_t)(E > 0 ? E : 1), sizeof(int32_t));
    for (int64_t t = 0; t < T; ++t)
        for (int32_t k = 0; k < K; ++k) {
            int e = slot_expert(t, k, K, expert_begin, E, idx, B, block_counts);
            if (e < 0) {
                row_map[t * K + k] = -1;
                continue;
            }
            int32_t r = offsets[e] + fill[e];
            fill[e] += 1;
            row_map[t * K + k] = r;
            row_src[r] = (int32_t)t;
            row_k[r] = k;
        }
    free(fill);
    return E > 0 ? (int64_t)offsets[E] : 0;
}

int64_t oracle_route(int64_t T, int32_t K, int64_t expert_begin, int32_t E,
                     const int64_t* idx, int32_t* counts, int32_t* offsets,
                     int32_t* row_map, int32_t* row_src, int32_t* row_k) {
    return oracle_route_padded(T, K, expert_begin, E, 0, NULL, idx, counts, offsets, row_map,
                               row_src, row_k);
}

int64_t oracle_compact_rows(int64_t T, int32_t B, const int32_t* block_counts,
                            int64_t row_bytes, const void* src, void* dst, int32_t to_padded) {
    /* the carrying rows, block by block, in row order: the n-th of them is
     * compact row n */
    int64_t n = 0;
    for (int64_t t = 0; t < T; ++t) {
        if (!carries_row(t, B, block_counts)) continue;
        if (to_padded)
            memcpy((char*)dst + t * row_bytes, (const char*)src + n * row_bytes, (size_t)row_bytes);
        else
            memcpy((char*)dst + n * row_bytes, (const char*)src + t * row_bytes, (size_t)row_bytes);
        n += 1;
    }
    return n;
}

void oracle_expand(int64_t R, int64_t H, int32_t eb, const void* x,
                   const int32_t* row_src, void* Xe) {
    for (int64_t r = 0; r < R; ++r)
        memcpy((char*)Xe + r * H * eb, (const char*)x + (int64_t)row_src[r] * H * eb,
               (size_t)(H * eb));
}

/* SwiGLU expert on one row; hbuf holds the I intermediate values. */
static void expert_mlp(int64_t H, int64_t I, int32_t dtype, const void* w1e,
                       const void* w2e, const void* x, int64_t x_off,
                       double* hbuf, double* out) {
    for (int64_t i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            double xv = elem(x, dtype, x_off + h);
            g += elem(w1e, dtype, i * H + h) * xv;
            u += elem(w1e, dtype, (I + i) * H + h) * xv;
        }
        hbuf[i] = oracle_silu(g) * u;
    }
    for (int64_t j = 0; j < H; ++j) {
        double o = 0.0;
        for (int64_t i = 0; i < I; ++i) o += elem(w2e, dtype, j * I + i) * hbuf[i];
        out[j] = o;
    }
}

void oracle_expert_mlp(int64_t H, int64_t I, int32_t dtype, const void* w1e,
                       const void* w2e, const void* x, double* out) {
    double* hbuf = (double*)malloc((size_t)I * sizeof(double));
    expert_mlp(H, I, dtype, w1e, w2e, x, 0, hbuf, out);
    free(hbuf);
}

void oracle_expert_rows(int64_t n, const int32_t* experts, const int64_t* tokens,
                        int64_t H, int64_t I, int32_t dtype, const void* x,
                        const void* w1, const void* w2, double* out,
                        int32_t nthreads) {
    const int64_t eb = elem_bytes(dtype);
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1) num_threads(oracle_threads(nthreads))
    for (i = 0; i < n; ++i) {
        double* hbuf = (double*)malloc((size_t)I * sizeof(double));
        const char* w1e = (const char*)w1 + (int64_t)experts[i] * 2 * I * H * eb;
        const char* w2e = (const char*)w2 + (int64_t)experts[i] * H * I * eb;
        expert_mlp(H, I, dtype, w1e, w2e, x, tokens[i] * H, hbuf, out + i * H);
        free(hbuf);
    }
}

void oracle_combine(int64_t T, int32_t K, int64_t H, int32_t dtype,
                    const int32_t* row_map, const float* w, const void* O,
                    double* y) {
    for (int64_t t = 0; t < T; ++t) {
        double* yt = y + t * H;
        for (int64_t j = 0; j < H; ++j) yt[j] = 0.0;
        for (int32_t k = 0; k < K; ++k) {
            int32_t r = row_map[t * K + k];
            if (r < 0) continue;
            double wk = w ? (double)w[t * K + k] : 1.0;
            for (int64_t j = 0; j < H; ++j) yt[j] += wk * elem(O, dtype, (int64_t)r * H + j);
        }
    }
}

void oracle_combine_epilogue(int64_t T, int32_t J, int64_t H, int32_t dtype,
                             const int32_t* src, const void* recv, double* y) {
    for (int64_t t = 0; t < T; ++t) {
        double* yt = y + t * H;
        for (int64_t h = 0; h < H; ++h) yt[h] = 0.0;
        for (int32_t j = 0; j < J; ++j) {
            const int32_t row = src[t * J + j];
            if (row < 0) continue;
            for (int64_t h = 0; h < H; ++h) yt[h] += elem(recv, dtype, (int64_t)row * H + h);
        }
    }
}

void oracle_forward(int64_t T, int32_t K, int64_t expert_begin, int32_t E,
                    int64_t H, int64_t I, int32_t dtype, const void* x,
                    const int64_t* idx, const float* w, const void* w1,
                    const void* w2, const int64_t* tokens, int64_t n_tokens,
                    double* y, int32_t nthreads) {
    const int64_t eb = elem_bytes(dtype);
    const int64_t n = tokens ? n_tokens : T;
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1) num_threads(oracle_threads(nthreads))
    for (i = 0; i < n; ++i) {
        const int64_t t = tokens ? tokens[i] : i;
        double* yt = y + i * H;
        double* hbuf = (double*)malloc((size_t)I * sizeof(double));
        double* o = (double*)malloc((size_t)H * sizeof(double));
        for (int64_t j = 0; j < H; ++j) yt[j] = 0.0;
        for (int32_t k = 0; k < K; ++k) {
            int e = local_expert(idx[t * K + k], expert_begin, E);
            if (e < 0) continue;
            const char* w1e = (const char*)w1 + (int64_t)e * 2 * I * H * eb;
            const char* w2e = (const char*)w2 + (int64_t)e * H * I * eb;
            expert_mlp(H, I, dtype, w1e, w2e, x, t * H, hbuf, o);
            double wk = w ? (double)w[t * K + k] : 1.0;
            for (int64_t j = 0; j < H; ++j) yt[j] += wk * o[j];
        }
        free(hbuf);
        free(o);
    }
}
