// C ABI of libtopreduce: argument checks, workspace layout, and the launch
// sequence of the hot path. Every entry point validates on the host and then
// only enqueues kernels on the caller's stream; nothing here allocates device
// memory or synchronises (moe_plan_stats excepted, by design).
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "tr_internal.h"

namespace {

thread_local char g_err[512] = "";

tr_status fail(tr_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

tr_status ok() {
  g_err[0] = '\0';
  return TR_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

tr_status check_desc(const tr_moe_desc* d) {
  if (!d) return fail(TR_EINVAL, "desc is NULL");
  if (d->T < 0) return fail(TR_EINVAL, "T must be >= 0 (got %lld)", (long long)d->T);
  if (d->K < 1 || d->K > tr::kMaxK) return fail(TR_EINVAL, "K must be in [1, %d] (got %d)", tr::kMaxK, d->K);
  if (d->E < 1 || d->E > tr::kMaxE) return fail(TR_EINVAL, "E must be in [1, %d] (got %d)", tr::kMaxE, d->E);
  if (d->H < 1 || d->I < 1) return fail(TR_EINVAL, "H and I must be >= 1");
  if (d->dtype != TR_BF16 && d->dtype != TR_F32) return fail(TR_EINVAL, "unknown dtype %d", d->dtype);
  if (d->idx_dtype != TR_IDX_I32 && d->idx_dtype != TR_IDX_I64)
    return fail(TR_EINVAL, "unknown idx_dtype %d", d->idx_dtype);
  const int32_t force = TR_FLAG_GEMM_FORCE_TILED | TR_FLAG_GEMM_FORCE_STREAM;
  if (d->flags & ~(force | TR_FLAG_NO_XE)) return fail(TR_EINVAL, "unknown flags 0x%x", d->flags);
  if ((d->flags & force) == force) return fail(TR_EINVAL, "both GEMM force flags set");
  // GEMM tiles address one expert's weights with 32-bit element offsets.
  if (d->H > (1 << 22) || d->I > (1 << 22) || 2 * d->H * d->I >= (int64_t(1) << 31))
    return fail(TR_EUNSUPPORTED, "H, I must be <= 2^22 and 2*H*I < 2^31");
  if (d->T > (int64_t(1) << 31) / d->K) return fail(TR_EUNSUPPORTED, "T*K must be < 2^31");
  if (d->expert_begin > (int64_t(1) << 62) || d->expert_begin < -(int64_t(1) << 62))
    return fail(TR_EINVAL, "expert_begin out of range");
  // rows of x, y, Xe and O move in 16-byte pieces
  if (d->H % 8) return fail(TR_EUNSUPPORTED, "H must be a multiple of 8 (got %lld)", (long long)d->H);
  // without an expanded buffer GEMM1 must be able to gather from x
  if ((d->flags & TR_FLAG_NO_XE) && !tr::gemm_can_gather(*d))
    return fail(TR_EUNSUPPORTED, "TR_FLAG_NO_XE needs bf16 and T * H * 2 < 2^31");
  return TR_OK;
}

struct Layout {
  int64_t R_cap;
  int blocks, rpb;
  size_t stats, counts, offsets, row_map, row_src, row_k, row_dst, tok_rest, scan_tmp, Xe, h, O,
      total;
};

Layout layout(const tr_moe_desc& d) {
  Layout L{};
  // one expanded row per local slot; a row may name the same expert twice
  L.R_cap = d.T * d.K;
  tr::route_scan_geometry(d.T, d.K, &L.blocks, &L.rpb);
  const size_t es = d.dtype == TR_BF16 ? 2 : 4;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = up(o + bytes); return at; };
  L.stats = take(16 * sizeof(int32_t));
  L.counts = take(sizeof(int32_t) * d.E);
  L.offsets = take(sizeof(int32_t) * (d.E + 1));
  L.row_map = take(sizeof(int32_t) * d.T * d.K);
  L.row_src = take(sizeof(int32_t) * L.R_cap);
  L.row_k = take(sizeof(int32_t) * L.R_cap);
  L.row_dst = take(sizeof(int32_t) * L.R_cap);
  L.tok_rest = take(sizeof(int32_t) * d.T);
  L.scan_tmp = take(sizeof(int32_t) * static_cast<size_t>(L.blocks) * (2 * d.E + 4));
  L.Xe = take((d.flags & TR_FLAG_NO_XE) ? 0 : es * (L.R_cap + tr::kRowPad) * d.H);
  L.h = take(es * (L.R_cap + tr::kRowPad) * d.I);
  L.O = take(es * L.R_cap * d.H);
  L.total = o;
  return L;
}

tr_status check_plan(const tr_moe_plan* p) {
  if (!p) return fail(TR_EINVAL, "plan is NULL");
  if (!p->ws) return fail(TR_EINVAL, "plan has no workspace (was moe_plan called?)");
  return check_desc(&p->d);
}

tr_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TR_EHIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace tr {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const int slot = dev < 64 ? dev : 63;
  int v = cache[slot].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cache[slot].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace tr

extern "C" {

size_t moe_workspace_size(const tr_moe_desc* desc) {
  if (check_desc(desc) != TR_OK) return 0;
  ok();
  return layout(*desc).total;
}

}  // extern "C"

namespace {

// moe_plan with optional padding blocks (B == 0: every row carries a token).
tr_status plan_rows(const tr_moe_desc* desc, const void* topk_idx, int32_t B,
                    const int32_t* block_counts, void* ws, size_t ws_bytes, hipStream_t stream,
                    tr_moe_plan* out) {
  tr_status s = check_desc(desc);
  if (s != TR_OK) return s;
  if (!out) return fail(TR_EINVAL, "out plan is NULL");
  if (!ws) return fail(TR_EINVAL, "workspace is NULL");
  if (!aligned(ws, kAlign)) return fail(TR_EINVAL, "workspace must be %zu-byte aligned", kAlign);
  const Layout L = layout(*desc);
  if (ws_bytes < L.total)
    return fail(TR_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
  const size_t isz = desc->idx_dtype == TR_IDX_I64 ? 8 : 4;
  if (desc->T > 0 && !topk_idx) return fail(TR_EINVAL, "topk_idx is NULL");
  if (topk_idx && !aligned(topk_idx, isz)) return fail(TR_EINVAL, "topk_idx misaligned");

  tr_moe_plan p;
  memset(&p, 0, sizeof p);
  p.d = *desc;
  p.R_cap = L.R_cap;
  p.ws = ws;
  p.ws_bytes = ws_bytes;
  char* b = static_cast<char*>(ws);
  p.stats = reinterpret_cast<int32_t*>(b + L.stats);
  p.counts = reinterpret_cast<int32_t*>(b + L.counts);
  p.offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  p.row_map = reinterpret_cast<int32_t*>(b + L.row_map);
  p.row_src = reinterpret_cast<int32_t*>(b + L.row_src);
  p.row_k = reinterpret_cast<int32_t*>(b + L.row_k);
  p.row_dst = reinterpret_cast<int32_t*>(b + L.row_dst);
  p.tok_rest = reinterpret_cast<int32_t*>(b + L.tok_rest);
  p.scan_tmp = reinterpret_cast<int32_t*>(b + L.scan_tmp);
  p.Xe = (desc->flags & TR_FLAG_NO_XE) ? nullptr : b + L.Xe;
  p.h = b + L.h;
  p.O = b + L.O;
  p.scan_blocks = L.blocks;
  p.scan_rows_per_block = L.rpb;
  p.block_rows = B;
  p.block_counts = block_counts;
  // T == 0 still runs the (one-block) scan so counts, offsets and stats are
  // defined as zeros.
  s = hip_status(tr::route_scan(p, topk_idx, stream), "moe_route_scan launch");
  if (s != TR_OK) return s;
  *out = p;
  return ok();
}

}  // namespace

extern "C" {

tr_status moe_plan(const tr_moe_desc* desc, const void* topk_idx, void* ws, size_t ws_bytes,
                   hipStream_t stream, tr_moe_plan* out) {
  return plan_rows(desc, topk_idx, 0, nullptr, ws, ws_bytes, stream, out);
}

tr_status moe_plan_padded(const tr_moe_desc* desc, const void* topk_idx, int32_t block_rows,
                          const int32_t* block_counts, void* ws, size_t ws_bytes,
                          hipStream_t stream, tr_moe_plan* out) {
  tr_status s = check_desc(desc);
  if (s != TR_OK) return s;
  if (block_rows < 1) return fail(TR_EINVAL, "block_rows must be >= 1 (got %d)", block_rows);
  if ((desc->T + block_rows - 1) / block_rows > tr::kMaxPadBlocks)
    return fail(TR_EUNSUPPORTED, "at most %d padding blocks (T / block_rows)", tr::kMaxPadBlocks);
  if (desc->T > 0 && (!block_counts || !aligned(block_counts, 4)))
    return fail(TR_EINVAL, "block_counts must be non-NULL and 4-byte aligned");
  return plan_rows(desc, topk_idx, block_rows, block_counts, ws, ws_bytes, stream, out);
}

tr_status moe_compact_rows(int64_t T, int32_t block_rows, const int32_t* block_counts,
                           int64_t row_bytes, const void* src, void* dst, int32_t to_padded,
                           int32_t* n_out, hipStream_t stream) {
  if (T < 0) return fail(TR_EINVAL, "T must be >= 0");
  // compact positions and row indices are 32-bit on the device
  if (T >= (int64_t{1} << 31)) return fail(TR_EUNSUPPORTED, "T must be < 2^31 (got %lld)", (long long)T);
  if (block_rows < 1) return fail(TR_EINVAL, "block_rows must be >= 1 (got %d)", block_rows);
  if ((T + block_rows - 1) / block_rows > tr::kMaxPadBlocks)
    return fail(TR_EUNSUPPORTED, "at most %d padding blocks (T / block_rows)", tr::kMaxPadBlocks);
  if (row_bytes < 4 || row_bytes % 4 != 0 || row_bytes > (int64_t{1} << 40))
    return fail(TR_EINVAL, "row_bytes must be a positive multiple of 4");
  if (T > 0 && row_bytes > (int64_t{1} << 62) / T)
    return fail(TR_EINVAL, "T * row_bytes overflows");
  if (to_padded != 0 && to_padded != 1) return fail(TR_EINVAL, "to_padded must be 0 or 1");
  if (n_out && !aligned(n_out, 4)) return fail(TR_EINVAL, "n_out misaligned");
  if (T > 0) {
    if (!block_counts || !aligned(block_counts, 4))
      return fail(TR_EINVAL, "block_counts must be non-NULL and 4-byte aligned");
    if (!src || !aligned(src, 4) || !dst || !aligned(dst, 4))
      return fail(TR_EINVAL, "src and dst must be non-NULL and 4-byte aligned");
  } else if (!n_out) {
    return ok();
  }
  return hip_status(tr::compact_rows(T, block_rows, block_counts, row_bytes, src, dst,
                                     to_padded != 0, n_out, stream),
                    "moe_compact_rows launch");
}

static tr_status check_buf(const void* p, const char* name, bool needed) {
  if (!needed) return TR_OK;
  if (!p) return fail(TR_EINVAL, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(TR_EINVAL, "%s must be 16-byte aligned", name);
  return TR_OK;
}

// The entry points that read or write the expanded buffer.
static tr_status check_has_xe(const tr_moe_plan* plan, const char* what) {
  if (plan->d.flags & TR_FLAG_NO_XE)
    return fail(TR_EUNSUPPORTED, "%s needs the expanded buffer (plan made with TR_FLAG_NO_XE)", what);
  return TR_OK;
}

tr_status moe_expand(const tr_moe_plan* plan, const void* x, hipStream_t stream) {
  tr_status s = check_plan(plan);
  if (s != TR_OK) return s;
  if ((s = check_has_xe(plan, "moe_expand")) != TR_OK) return s;
  const bool any = plan->d.T > 0;
  if ((s = check_buf(x, "x", any)) != TR_OK) return s;
  if (!any) return ok();
  return hip_status(tr::expand(*plan, x, stream), "moe_expand launch");
}

tr_status moe_grouped_gemm(const tr_moe_plan* plan, const void* w1, const void* w2,
                           hipStream_t stream) {
  tr_status s = check_plan(plan);
  if (s != TR_OK) return s;
  if ((s = check_has_xe(plan, "moe_grouped_gemm")) != TR_OK) return s;
  const bool any = plan->d.T > 0;
  if ((s = check_buf(w1, "w1", any)) != TR_OK) return s;
  if ((s = check_buf(w2, "w2", any)) != TR_OK) return s;
  if (!any) return ok();
  return hip_status(tr::grouped_gemm(*plan, w1, w2, tr::kGemmUp | tr::kGemmDown, stream),
                    "moe_grouped_gemm launch");
}

tr_status moe_grouped_gemm_up(const tr_moe_plan* plan, const void* w1, hipStream_t stream) {
  tr_status s = check_plan(plan);
  if (s != TR_OK) return s;
  if ((s = check_has_xe(plan, "moe_grouped_gemm_up")) != TR_OK) return s;
  const bool any = plan->d.T > 0;
  if ((s = check_buf(w1, "w1", any)) != TR_OK) return s;
  if (!any) return ok();
  return hip_status(tr::grouped_gemm(*plan, w1, nullptr, tr::kGemmUp, stream),
                    "moe_grouped_gemm_up launch");
}

tr_status moe_grouped_gemm_up_x(const tr_moe_plan* plan, const void* x, const void* w1,
                                hipStream_t stream) {
  tr_status s = check_plan(plan);
  if (s != TR_OK) return s;
  const bool any = plan->d.T > 0;
  if ((s = check_buf(x, "x", any)) != TR_OK) return s;
  if ((s = check_buf(w1, "w1", any)) != TR_OK) return s;
  if (!any) return ok();
  if (plan->d.dtype == TR_BF16 && !tr::gemm_can_gather(plan->d)) {
    // bf16 with x past 2 GiB: expand first, then GEMM1 over Xe
    if ((s = hip_status(tr::expand(*plan, x, stream), "moe_expand launch")) != TR_OK) return s;
    return hip_status(tr::grouped_gemm(*plan, w1, nullptr, tr::kGemmUp, stream),
                      "moe_grouped_gemm_up launch");
  }
  return hip_status(tr::grouped_gemm(*plan, w1, nullptr, tr::kGemmUp, stream, x),
                    "moe_grouped_gemm_up_x launch");
}

tr_status moe_grouped_gemm_down(const tr_moe_plan* plan, const void* w2, hipStream_t stream) {
  tr_status s = check_plan(plan);
  if (s != TR_OK) return s;
  const bool any = plan->d.T > 0;
  if ((s = check_buf(w2, "w2", any)) != TR_OK) return s;
  if (!any) return ok();
  return hip_status(tr::grouped_gemm(*plan, nullptr, w2, tr::kGemmDown, stream),
                    "moe_grouped_gemm_down launch");
}

tr_status moe_grouped_gemm_down_y(const tr_moe_plan* plan, const void* w2,
                                  const float* topk_weights, void* y, hipStream_t stream) {
  tr_status s = check_plan(plan);
  if (s != TR_OK) return s;
  const bool any = plan->d.T > 0;
  if ((s = check_buf(w2, "w2", any)) != TR_OK) return s;
  if ((s = check_buf(y, "y", any)) != TR_OK) return s;
  if (topk_weights && !aligned(topk_weights, 4)) return fail(TR_EINVAL, "topk_weights misaligned");
  if (!tr::gemm_can_gather(plan->d))
    return fail(TR_EUNSUPPORTED, "moe_grouped_gemm_down_y needs bf16 and T * H * 2 < 2^31");
  if (!any) return ok();
  return hip_status(tr::grouped_gemm(*plan, nullptr, w2, tr::kGemmDown, stream, nullptr,
                                     topk_weights, y),
                    "moe_grouped_gemm_down_y launch");
}

tr_status moe_combine_reduce_multi(const tr_moe_plan* plan, const float* topk_weights, void* y,
                                   hipStream_t stream) {
  tr_status s = check_plan(plan);
  if (s != TR_OK) return s;
  const bool any = plan->d.T > 0;
  if ((s = check_buf(y, "y", any)) != TR_OK) return s;
  if (topk_weights && !aligned(topk_weights, 4)) return fail(TR_EINVAL, "topk_weights misaligned");
  if (!any) return ok();
  return hip_status(tr::combine_reduce(*plan, nullptr, topk_weights, y, stream, true),
                    "moe_combine_reduce_multi launch");
}

tr_status moe_combine_reduce(const tr_moe_plan* plan, const void* expert_out,
                             const float* topk_weights, void* y, hipStream_t stream) {
  tr_status s = check_plan(plan);
  if (s != TR_OK) return s;
  const bool any = plan->d.T > 0;
  if ((s = check_buf(y, "y", any)) != TR_OK) return s;
  if (expert_out && !aligned(expert_out, 16)) return fail(TR_EINVAL, "expert_out must be 16-byte aligned");
  if (topk_weights && !aligned(topk_weights, 4)) return fail(TR_EINVAL, "topk_weights misaligned");
  if (!any) return ok();
  return hip_status(tr::combine_reduce(*plan, expert_out, topk_weights, y, stream),
                    "moe_combine_reduce launch");
}

tr_status moe_forward(const tr_moe_plan* plan, const void* x, const float* topk_weights,
                      const void* w1, const void* w2, void* y, hipStream_t stream) {
  tr_status s = check_plan(plan);
  if (s != TR_OK) return s;
  const bool any = plan->d.T > 0;
  if ((s = check_buf(x, "x", any)) != TR_OK) return s;
  if ((s = check_buf(w1, "w1", any)) != TR_OK) return s;
  if ((s = check_buf(w2, "w2", any)) != TR_OK) return s;
  if ((s = check_buf(y, "y", any)) != TR_OK) return s;
  if (topk_weights && !aligned(topk_weights, 4)) return fail(TR_EINVAL, "topk_weights misaligned");
  if (!any) return ok();
  if (tr::gemm_can_gather(plan->d)) {
    // GEMM1 reads x through the route table (no expand pass, Xe unused);
    // GEMM2 writes received rows with one local slot straight to y, and the
    // reduce completes the others
    bool y_done = false;
    if ((s = hip_status(tr::grouped_gemm(*plan, w1, w2, tr::kGemmUp | tr::kGemmDown, stream, x,
                                         topk_weights, y, &y_done),
                        "moe_grouped_gemm launch")) != TR_OK)
      return s;
    if (y_done) return ok();   // a decode batch: GEMM2 ran the reduce
    return hip_status(tr::combine_reduce(*plan, nullptr, topk_weights, y, stream, true),
                      "moe_combine_reduce launch");
  } else if (plan->d.dtype == TR_F32) {
    // fp32: GEMM1 reads x through the route table too (no expand pass);
    // GEMM2 writes O for every row and the reduce takes them all
    if ((s = hip_status(tr::grouped_gemm(*plan, w1, w2, tr::kGemmUp | tr::kGemmDown, stream, x),
                        "moe_grouped_gemm launch")) != TR_OK)
      return s;
  } else {
    if ((s = hip_status(tr::expand(*plan, x, stream), "moe_expand launch")) != TR_OK) return s;
    if ((s = hip_status(tr::grouped_gemm(*plan, w1, w2, tr::kGemmUp | tr::kGemmDown, stream),
                        "moe_grouped_gemm launch")) != TR_OK)
      return s;
  }
  return hip_status(tr::combine_reduce(*plan, nullptr, topk_weights, y, stream),
                    "moe_combine_reduce launch");
}

tr_status moe_combine_epilogue(int64_t T, int32_t J, int64_t H, tr_dtype dtype,
                               const int32_t* src, const void* recv, int64_t n_recv, void* y,
                               hipStream_t stream) {
  if (T < 0) return fail(TR_EINVAL, "T must be >= 0");
  if (J < 1 || J > 65536) return fail(TR_EINVAL, "J must be in [1, 65536]");
  if (H < 8 || H % 8 != 0 || H > (int64_t{1} << 22))
    return fail(TR_EUNSUPPORTED, "H must be a positive multiple of 8 (at most 2^22)");
  if (dtype != TR_BF16 && dtype != TR_F32) return fail(TR_EINVAL, "unknown dtype");
  if (n_recv < 0 || n_recv > INT32_MAX) return fail(TR_EINVAL, "n_recv must be in [0, 2^31)");
  if (T * static_cast<int64_t>(J) >= (int64_t{1} << 31)) return fail(TR_EINVAL, "T * J too large");
  if (T == 0) return ok();
  if (!src || !aligned(src, 4)) return fail(TR_EINVAL, "src must be non-NULL and 4-byte aligned");
  tr_status s;
  if ((s = check_buf(y, "y", true)) != TR_OK) return s;
  if (n_recv > 0 && (s = check_buf(recv, "recv", true)) != TR_OK) return s;
  return hip_status(tr::combine_epilogue(T, J, H, dtype == TR_BF16, src, recv, n_recv, y, stream),
                    "moe_combine_epilogue launch");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free forward: plan + forward in a workspace the library holds
// itself, for callers that cannot allocate device memory (code under HIP graph
// capture, serving loops, harnesses that forbid allocation).
// ---------------------------------------------------------------------------
namespace {

// The workspace of moe_forward_noalloc. Each device the library runs on holds
// its own copy from module load until the process ends. In host code this
// name is only a stand-in: kernels get the device address that
// hipGetSymbolAddress returns for it (noalloc_scratch_ptr).
static __device__ __align__(256) unsigned char scratch[TR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch array, looked up once per device
// with that device current; NULL (and *err set) if the lookup fails.
void* noalloc_scratch_ptr(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (*err != hipSuccess) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

tr_status moe_forward_noalloc(const tr_moe_desc* desc, const void* topk_idx, const void* x,
                              const float* topk_weights, const void* w1, const void* w2,
                              void* y, hipStream_t stream) {
  tr_status s = check_desc(desc);
  if (s != TR_OK) return s;
  tr_moe_desc d = *desc;
  // bf16 gathers x inside GEMM1, so the expanded rows are never needed
  if (d.dtype == TR_BF16 && tr::gemm_can_gather(d)) d.flags |= TR_FLAG_NO_XE;
  const size_t need = layout(d).total;
  if (need > static_cast<size_t>(TR_NOALLOC_SCRATCH_BYTES))
    return fail(TR_EUNSUPPORTED,
                "moe_forward_noalloc: this batch needs %zu bytes of workspace, the library's "
                "static scratch holds %zu (use moe_plan + moe_forward with a caller workspace)",
                need, static_cast<size_t>(TR_NOALLOC_SCRATCH_BYTES));
  const bool any = d.T > 0;
  if ((s = check_buf(x, "x", any)) != TR_OK) return s;
  if ((s = check_buf(w1, "w1", any)) != TR_OK) return s;
  if ((s = check_buf(w2, "w2", any)) != TR_OK) return s;
  if ((s = check_buf(y, "y", any)) != TR_OK) return s;
  if (topk_weights && !aligned(topk_weights, 4)) return fail(TR_EINVAL, "topk_weights misaligned");
  hipError_t e = hipSuccess;
  void* ws = noalloc_scratch_ptr(&e);
  if (!ws) return hip_status(e, "moe_forward_noalloc: address of the static scratch");
  tr_moe_plan p;
  if ((s = plan_rows(&d, topk_idx, 0, nullptr, ws, need, stream, &p)) != TR_OK) return s;
  return moe_forward(&p, x, topk_weights, w1, w2, y, stream);
}

tr_status moe_plan_stats(const tr_moe_plan* plan, int32_t* host_out, hipStream_t stream) {
  tr_status s = check_plan(plan);
  if (s != TR_OK) return s;
  if (!host_out) return fail(TR_EINVAL, "host_out is NULL");
  hipError_t e = hipMemcpyAsync(host_out, plan->stats, 4 * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return hip_status(e, "moe_plan_stats");
}

const char* moe_last_error(void) { return g_err; }

int32_t moe_abi_version(void) { return TR_ABI_VERSION; }

}  // extern "C"
