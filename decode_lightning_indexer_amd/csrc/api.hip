// C ABI of the sparse-decode library: host-side checks, launch dispatch and
// the whole-step orchestration.  Every check happens before anything is
// enqueued, so a nonzero status means the stream is untouched.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "ess_host.h"
#include "ess_internal.h"
#include "fp8_entry.h"

namespace {

thread_local std::string g_err;

ess_status fail(ess_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

}  // namespace

ess_status ess::host_fail(ess_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

// The largest dynamic LDS size set so far for each (kernel, device): the
// attribute call runs only when a launch needs more.
hipError_t ess::ensure_dyn_lds(const void* fn, int bytes) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> set;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  int& have = set[{fn, dev}];
  if (bytes <= have) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) have = bytes;
  return e;
}

namespace {

ess_status hip_fail(hipError_t e, const char* what) {
  return fail(ESS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define ESS_NONNULL(p) \
  if (!(p)) return fail(ESS_ERR_INVALID, "%s: %s is NULL", fn, #p)

ess_status check_dims(const ess_dims* d, const char* fn) {
  if (!d) return fail(ESS_ERR_INVALID, "%s: dims is NULL", fn);
  if (d->batch < 1 || d->mtp < 1 || d->ctx_len < 1 || d->idx_heads < 1 ||
      d->idx_dim < 1 || d->mla_heads < 1 || d->topk < 1 || d->pool_slots < 1)
    return fail(ESS_ERR_INVALID, "%s: every size in dims must be >= 1", fn);
  if (d->lat_dim != ess::kLat || d->v_dim != ess::kVal)
    return fail(ESS_ERR_UNSUPPORTED, "%s: lat_dim must be 576 and v_dim 512",
                fn);
  if (d->mtp > 4)
    return fail(ESS_ERR_UNSUPPORTED, "%s: mtp above 4", fn);
  if (!std::isfinite(d->softmax_scale))
    return fail(ESS_ERR_INVALID, "%s: softmax_scale is not finite", fn);
  if (d->ctx_len > (1 << 28))
    return fail(ESS_ERR_UNSUPPORTED, "%s: ctx_len above 2^28", fn);
  return ESS_OK;
}

ess_status check_indexer(const ess_dims* d, const char* fn) {
  if (d->idx_dim != 64 && d->idx_dim != 128)
    return fail(ESS_ERR_UNSUPPORTED, "%s: idx_dim must be 64 or 128", fn);
  if (d->idx_heads % 16 != 0 || d->mtp * d->idx_heads > 128)
    return fail(ESS_ERR_UNSUPPORTED,
                "%s: idx_heads must be a multiple of 16 with mtp*idx_heads <= 128",
                fn);
  return ESS_OK;
}

ess_status check_topk(const ess_dims* d, int k, int n_tok, const char* fn) {
  if (k < 1 || k > ess::kMaxTopk)
    return fail(ESS_ERR_UNSUPPORTED, "%s: k must be in [1, %d]", fn,
                ess::kMaxTopk);
  if (n_tok < 1 || n_tok > d->mtp)
    return fail(ESS_ERR_INVALID, "%s: n_tok must be in [1, mtp]", fn);
  return ESS_OK;
}

ess_status check_update(const ess_dims* d, int k, int n_tok, const char* fn) {
  ess_status s = check_topk(d, k, n_tok, fn);
  if (s != ESS_OK) return s;
  if ((int64_t)n_tok * k > d->pool_slots)
    return fail(ESS_ERR_CAPACITY,
                "%s: n_tok*k = %lld exceeds pool_slots = %d", fn,
                (long long)n_tok * k, d->pool_slots);
  if ((int64_t)n_tok * k > ess::kMaxTopk)
    return fail(ESS_ERR_UNSUPPORTED, "%s: n_tok*k above %d", fn,
                ess::kMaxTopk);
  if (d->pool_slots > ess::kMaxPoolSlots)
    return fail(ESS_ERR_UNSUPPORTED, "%s: pool_slots above %d", fn,
                ess::kMaxPoolSlots);
  return ESS_OK;
}

ess_status check_mla(const ess_dims* d, const char* fn) {
  if (d->mla_heads % 16 != 0)
    return fail(ESS_ERR_UNSUPPORTED, "%s: mla_heads must be a multiple of 16",
                fn);
  if (d->topk > ess::kMaxTopk)
    return fail(ESS_ERR_UNSUPPORTED, "%s: topk above %d", fn, ess::kMaxTopk);
  return ESS_OK;
}

// Events that order one call's streams against each other.  Each host
// thread has its own pool: a call records and waits on its events while it
// enqueues (a wait takes the event's state at that moment), so a later call
// on the same thread may reuse them, and calls on different threads never
// share one.
thread_local std::vector<hipEvent_t> g_events;

ess_status get_events(size_t n, hipEvent_t** out) {
  while (g_events.size() < n) {
    hipEvent_t e;
    hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (r != hipSuccess) return hip_fail(r, "hipEventCreateWithFlags");
    g_events.push_back(e);
  }
  *out = g_events.data();
  return ESS_OK;
}

// Workspace layout: the attention's partials, then the top-k levels' lists
// (sized for the step's top-k and for the first fill's top-C), then each
// token's selection in position order (position, rank, slot) for the
// residency update of a step with several query tokens.
size_t attn_region(const ess_dims& d) {
  return ess::align_up(ess::sparse_mla_ws_bytes(d), 256);
}
size_t topk_region(const ess_dims& d) {
  const size_t a = ess::topk_ws_bytes(d, d.topk, d.mtp);
  const size_t b = ess::topk_ws_bytes(d, d.pool_slots, 1);
  return ess::align_up(a > b ? a : b, 256);
}
size_t lists_region(const ess_dims& d) {
  return ess::align_up((size_t)d.batch * d.mtp * d.topk * 3 * sizeof(int32_t), 256);
}
size_t ws_total(const ess_dims& d) {
  return attn_region(d) + topk_region(d) + lists_region(d);
}

}  // namespace

extern "C" {

size_t ess_workspace_bytes(const ess_dims* d) {
  if (check_dims(d, "ess_workspace_bytes") != ESS_OK) return 0;
  return ws_total(*d);
}

size_t ess_lru_state_bytes(const ess_dims* d) {
  if (check_dims(d, "ess_lru_state_bytes") != ESS_OK) return 0;
  return ess::lru_bytes_per_req(d->pool_slots) * (size_t)d->batch;
}

ess_status ess_pool_reset(const ess_dims* d, int32_t* cache_slots,
                          int32_t* slot_pos, void* lru_state,
                          hipStream_t stream) {
  const char* fn = "ess_pool_reset";
  ess_status s = check_dims(d, fn);
  if (s != ESS_OK) return s;
  ESS_NONNULL(cache_slots);
  ESS_NONNULL(slot_pos);
  ESS_NONNULL(lru_state);
  hipError_t e = ess::launch_pool_reset(*d, cache_slots, slot_pos, lru_state,
                                        stream);
  return e == hipSuccess ? ESS_OK : hip_fail(e, fn);
}

ess_status ess_pool_status(const ess_dims* d, const void* lru_state,
                           int32_t* status, hipStream_t stream) {
  const char* fn = "ess_pool_status";
  ess_status s = check_dims(d, fn);
  if (s != ESS_OK) return s;
  ESS_NONNULL(lru_state);
  ESS_NONNULL(status);
  hipError_t e = ess::launch_pool_status(*d, lru_state, status, stream);
  return e == hipSuccess ? ESS_OK : hip_fail(e, fn);
}

ess_status ess_copy_async(void* dst, const void* src, size_t bytes,
                          hipStream_t stream) {
  const char* fn = "ess_copy_async";
  ESS_NONNULL(dst);
  ESS_NONNULL(src);
  if (bytes == 0) return ESS_OK;
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDefault, stream);
  return e == hipSuccess ? ESS_OK : hip_fail(e, fn);
}

ess_status ess_thread_release(void) {
  hipError_t first = hipSuccess;
  for (hipEvent_t e : g_events) {
    const hipError_t r = hipEventDestroy(e);
    if (first == hipSuccess) first = r;
  }
  g_events.clear();
  g_events.shrink_to_fit();
  return first == hipSuccess ? ESS_OK : hip_fail(first, "ess_thread_release");
}

ess_status ess_index_scores(const ess_dims* d, const uint8_t* q_fp8,
                            const float* w, const uint8_t* k_fp8,
                            const int32_t* n_vis, float* scores,
                            hipStream_t stream) {
  const char* fn = "ess_index_scores";
  ess_status s = check_dims(d, fn);
  if (s != ESS_OK) return s;
  if ((s = check_indexer(d, fn)) != ESS_OK) return s;
  ESS_NONNULL(q_fp8);
  ESS_NONNULL(w);
  ESS_NONNULL(k_fp8);
  ESS_NONNULL(n_vis);
  ESS_NONNULL(scores);
  hipError_t e = ess::launch_index_scores(*d, q_fp8, w, k_fp8, n_vis, scores,
                                          stream);
  return e == hipSuccess ? ESS_OK : hip_fail(e, fn);
}

ess_status ess_topk_lookup(const ess_dims* d, int32_t k, int32_t n_tok,
                           const float* scores, const int32_t* n_vis,
                           const int32_t* cache_slots, int32_t* sel_pos,
                           int32_t* sel_slot, int32_t* n_sel, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  const char* fn = "ess_topk_lookup";
  ess_status s = check_dims(d, fn);
  if (s != ESS_OK) return s;
  if ((s = check_topk(d, k, n_tok, fn)) != ESS_OK) return s;
  ESS_NONNULL(scores);
  ESS_NONNULL(n_vis);
  ESS_NONNULL(cache_slots);
  ESS_NONNULL(sel_pos);
  ESS_NONNULL(sel_slot);
  ESS_NONNULL(n_sel);
  const size_t need = ess::topk_ws_bytes(*d, k, n_tok);
  if (need > 0 && ws && (reinterpret_cast<uintptr_t>(ws) & 15))
    return fail(ESS_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(ESS_ERR_NOMEM,
                "%s: rows of %d keys select over a workspace of %zu bytes "
                "(have %zu)", fn, d->ctx_len, need, ws ? ws_bytes : 0);
  hipError_t e = ess::launch_topk(*d, k, n_tok, scores, n_vis, cache_slots,
                                  sel_pos, sel_slot, n_sel,
                                  need > 0 ? ws : nullptr, stream);
  return e == hipSuccess ? ESS_OK : hip_fail(e, fn);
}

ess_status ess_pool_update(const ess_dims* d, int32_t k, int32_t n_tok,
                           const int32_t* sel_pos, const int32_t* n_sel,
                           int32_t* cache_slots, int32_t* slot_pos,
                           void* lru_state, int32_t* miss_pos,
                           int32_t* miss_slot, int32_t* n_miss,
                           int32_t* n_evict, int32_t* row_dst,
                           int32_t* sel_slot_post, hipStream_t stream) {
  const char* fn = "ess_pool_update";
  ess_status s = check_dims(d, fn);
  if (s != ESS_OK) return s;
  if ((s = check_update(d, k, n_tok, fn)) != ESS_OK) return s;
  ESS_NONNULL(sel_pos);
  ESS_NONNULL(n_sel);
  ESS_NONNULL(cache_slots);
  ESS_NONNULL(slot_pos);
  ESS_NONNULL(lru_state);
  ESS_NONNULL(miss_pos);
  ESS_NONNULL(miss_slot);
  ESS_NONNULL(n_miss);
  ESS_NONNULL(n_evict);
  ESS_NONNULL(row_dst);
  ESS_NONNULL(sel_slot_post);
  hipError_t e = ess::launch_pool_update(*d, k, n_tok, sel_pos, n_sel,
                                         cache_slots, slot_pos, lru_state,
                                         miss_pos, miss_slot, n_miss, n_evict,
                                         row_dst, sel_slot_post, stream);
  return e == hipSuccess ? ESS_OK : hip_fail(e, fn);
}

static ess_status sparse_mla_call(const char* fn, const ess_dims* d,
                                  const uint16_t* q_abs, const int32_t* sel_pos,
                                  const int32_t* sel_src, const int32_t* row_dst,
                                  const int32_t* n_sel, uint16_t* pool,
                                  const uint16_t* host_view,
                                  const uint8_t* entry_view, float* out,
                                  float* lse, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  ess_status s = check_dims(d, fn);
  if (s != ESS_OK) return s;
  if ((s = check_mla(d, fn)) != ESS_OK) return s;
  ESS_NONNULL(q_abs);
  ESS_NONNULL(sel_pos);
  ESS_NONNULL(sel_src);
  ESS_NONNULL(n_sel);
  ESS_NONNULL(pool);
  if (!host_view && !entry_view)
    return fail(ESS_ERR_INVALID, "%s: NULL host store", fn);
  if (entry_view && (reinterpret_cast<uintptr_t>(entry_view) & 15))
    return fail(ESS_ERR_INVALID, "%s: entry_view must be 16-byte aligned", fn);
  ESS_NONNULL(out);
  ESS_NONNULL(ws);
  if (reinterpret_cast<uintptr_t>(ws) & 15)
    return fail(ESS_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
  const size_t need = ess::sparse_mla_ws_bytes(*d);
  if (ws_bytes < need)
    return fail(ESS_ERR_NOMEM, "%s: workspace of %zu bytes, need %zu", fn,
                ws_bytes, need);
  hipError_t e = ess::launch_sparse_mla(*d, q_abs, sel_pos, sel_src, row_dst,
                                        n_sel, pool, host_view, out, lse, ws,
                                        stream, 0, entry_view);
  return e == hipSuccess ? ESS_OK : hip_fail(e, fn);
}

ess_status ess_sparse_mla_decode(const ess_dims* d, const uint16_t* q_abs,
                                 const int32_t* sel_pos,
                                 const int32_t* sel_src,
                                 const int32_t* row_dst, const int32_t* n_sel,
                                 uint16_t* pool, const uint16_t* host_view,
                                 float* out, float* lse, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  const char* fn = "ess_sparse_mla_decode";
  ESS_NONNULL(host_view);
  return sparse_mla_call(fn, d, q_abs, sel_pos, sel_src, row_dst, n_sel, pool,
                         host_view, nullptr, out, lse, ws, ws_bytes, stream);
}

ess_status ess_sparse_mla_decode_noalloc(const ess_dims* d, const uint16_t* q_abs,
                                         const int32_t* sel_pos,
                                         const int32_t* sel_src,
                                         const int32_t* row_dst,
                                         const int32_t* n_sel, uint16_t* pool,
                                         const uint16_t* host_view, float* out,
                                         float* lse, hipStream_t stream) {
  const char* fn = "ess_sparse_mla_decode_noalloc";
  ess_status s = check_dims(d, fn);
  if (s != ESS_OK) return s;
  if ((s = check_mla(d, fn)) != ESS_OK) return s;
  ESS_NONNULL(q_abs);
  ESS_NONNULL(sel_pos);
  ESS_NONNULL(sel_src);
  ESS_NONNULL(n_sel);
  ESS_NONNULL(pool);
  ESS_NONNULL(host_view);
  ESS_NONNULL(out);
  const size_t need = ess::sparse_mla_ws_bytes(*d);
  if (need > ess::kNoAllocScratchBytes)
    return fail(ESS_ERR_NOMEM,
                "%s: these dims need %zu bytes of scratch; the fixed scratch "
                "array holds %zu (use ess_sparse_mla_decode with a workspace)",
                fn, need, ess::kNoAllocScratchBytes);
  hipError_t e = ess::launch_sparse_mla_noalloc(*d, q_abs, sel_pos, sel_src, row_dst,
                                                n_sel, pool, host_view, out, lse,
                                                stream);
  return e == hipSuccess ? ESS_OK : hip_fail(e, fn);
}

ess_status ess_sparse_mla_decode_entries(
    const ess_dims* d, const uint16_t* q_abs, const int32_t* sel_pos,
    const int32_t* sel_src, const int32_t* row_dst, const int32_t* n_sel,
    uint16_t* pool, const uint8_t* entry_view, float* out, float* lse,
    void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "ess_sparse_mla_decode_entries";
  ESS_NONNULL(entry_view);
  return sparse_mla_call(fn, d, q_abs, sel_pos,
                         sel_src, row_dst, n_sel, pool, nullptr, entry_view,
                         out, lse, ws, ws_bytes, stream);
}

ess_status ess_miss_copy(const ess_dims* d, int32_t list_stride,
                         const int32_t* miss_pos, const int32_t* miss_slot,
                         const int32_t* n_miss, const uint16_t* host_view,
                         uint16_t* pool, hipStream_t stream) {
  const char* fn = "ess_miss_copy";
  ess_status s = check_dims(d, fn);
  if (s != ESS_OK) return s;
  if (list_stride < 1)
    return fail(ESS_ERR_INVALID, "%s: list_stride must be >= 1", fn);
  ESS_NONNULL(miss_pos);
  ESS_NONNULL(miss_slot);
  ESS_NONNULL(n_miss);
  ESS_NONNULL(host_view);
  ESS_NONNULL(pool);
  hipError_t e = ess::launch_miss_copy(*d, list_stride, miss_pos, miss_slot,
                                       n_miss, host_view, pool, stream);
  return e == hipSuccess ? ESS_OK : hip_fail(e, fn);
}

ess_status ess_miss_copy_entries(const ess_dims* d, int32_t list_stride,
                                 const int32_t* miss_pos,
                                 const int32_t* miss_slot,
                                 const int32_t* n_miss,
                                 const uint8_t* entry_view, uint16_t* pool,
                                 hipStream_t stream) {
  const char* fn = "ess_miss_copy_entries";
  ess_status s = check_dims(d, fn);
  if (s != ESS_OK) return s;
  if (list_stride < 1)
    return fail(ESS_ERR_INVALID, "%s: list_stride must be >= 1", fn);
  ESS_NONNULL(miss_pos);
  ESS_NONNULL(miss_slot);
  ESS_NONNULL(n_miss);
  ESS_NONNULL(entry_view);
  ESS_NONNULL(pool);
  if (reinterpret_cast<uintptr_t>(entry_view) & 15)
    return fail(ESS_ERR_INVALID, "%s: entry_view must be 16-byte aligned", fn);
  hipError_t e = ess::launch_entry_copy(*d, list_stride, miss_pos, miss_slot,
                                        n_miss, entry_view, pool, stream);
  return e == hipSuccess ? ESS_OK : hip_fail(e, fn);
}

static ess_status check_layer(const ess_layer_io& io, int mode, int l) {
  const char* fn = "ess_decode_step";
  if (!io.q_idx || !io.w_idx || !io.k_idx || (!io.host_view && !io.host_entries) || !io.pool ||
      !io.cache_slots || !io.slot_pos || !io.lru_state || !io.scores ||
      !io.sel_pos || !io.sel_slot || !io.n_sel || !io.row_dst ||
      !io.sel_slot_post || !io.miss_pos || !io.miss_slot || !io.n_miss ||
      !io.n_evict)
    return fail(ESS_ERR_INVALID, "%s: layer %d has a NULL buffer", fn, l);
  if (mode != ESS_MODE_FILL && (!io.q_abs || !io.out || !io.ws))
    return fail(ESS_ERR_INVALID, "%s: layer %d has a NULL attention buffer",
                fn, l);
  if (io.host_entries && (reinterpret_cast<uintptr_t>(io.host_entries) & 15))
    return fail(ESS_ERR_INVALID, "%s: layer %d host_entries must be 16-byte aligned",
                fn, l);
  if (io.tail_rows && mode == ESS_MODE_FILL)
    return fail(ESS_ERR_INVALID,
                "%s: layer %d: the first fill reads the host store and precedes the tail",
                fn, l);
  if (io.tail_rows && (io.tail_block < 1 || !io.tail_start))
    return fail(ESS_ERR_INVALID, "%s: layer %d: tail_block must be >= 1 and tail_start set",
                fn, l);
  if (io.ws && (reinterpret_cast<uintptr_t>(io.ws) & 15))
    return fail(ESS_ERR_INVALID, "%s: layer %d workspace must be 16-byte aligned",
                fn, l);
  return ESS_OK;
}

// Scores, top-k and pool update of one layer on one stream; tws: the
// layer's top-k region of its workspace (nullptr: one workgroup per row);
// lws: its position-list region (nullptr: none).  beside: the selection
// runs beside other kernels (the prefetch side stream), so long rows select
// in levels rather than split over workgroups that wait for one another
// (measured over 16 layers of 64K x 32: split 4880 against levels 4610 us
// per prefetch step, while inline the split is faster, 5230 against 5280).
static hipError_t enqueue_select(const ess_dims& d, const ess_layer_io& io,
                                 const int32_t* n_vis, int k, int n_tok,
                                 void* tws, void* lws, hipStream_t st,
                                 bool beside = false) {
  // A selection split over several workgroups per row has its control
  // words cleared by the indexer, which runs just before it on this stream.
  ess::ClearSpec clr{nullptr, 0, 0, 0};
  const bool cleared = !beside && ess::split_clear(d, k, n_tok, tws, &clr);
  hipError_t e = ess::launch_index_scores(d, io.q_idx, io.w_idx, io.k_idx,
                                          n_vis, io.scores, st, clr);
  if (e != hipSuccess) return e;
  if (ess::select_update_fits(d, k, n_tok))
    return ess::launch_select_update(d, k, io.scores, n_vis, io.cache_slots,
                                     io.sel_pos, io.sel_slot, io.n_sel,
                                     io.slot_pos, io.lru_state, io.miss_pos,
                                     io.miss_slot, io.n_miss, io.n_evict,
                                     io.row_dst, io.sel_slot_post, tws, st,
                                     cleared, !beside);
  // Several tokens: the top-k leaves each token's winners in position order
  // (when it ranks them from a compact list) and the update merges those
  // lists instead of sorting the union.
  ess::PosLists pl{nullptr, nullptr, nullptr};
  if (lws && (size_t)n_tok * k <= (size_t)d.mtp * d.topk &&
      ess::topk_pos_lists_fit(d, k, tws != nullptr)) {
    int32_t* base = static_cast<int32_t*>(lws);
    const size_t n = (size_t)d.batch * n_tok * k;
    pl = ess::PosLists{base, base + n, base + 2 * n};
  }
  e = ess::launch_topk(d, k, n_tok, io.scores, n_vis, io.cache_slots,
                       io.sel_pos, io.sel_slot, io.n_sel, tws, st, pl, cleared,
                       !beside);
  if (e != hipSuccess) return e;
  // The update takes each row's pre-update slot from the top-k's lookup.
  return ess::launch_pool_update(d, k, n_tok, io.sel_pos, io.n_sel,
                                 io.cache_slots, io.slot_pos, io.lru_state,
                                 io.miss_pos, io.miss_slot, io.n_miss,
                                 io.n_evict, io.row_dst, io.sel_slot_post, st,
                                 io.sel_slot, pl);
}

// Gather + attention of one selected layer: the attention reads each miss
// from host memory into its tile and writes it to its slot from there, so
// the host reads run under the attention's own work.
// Gather + attention of one selected layer: the attention reads each miss
// from host memory (a bf16 row, or a 656-byte fp8 entry it dequantizes in
// the tile) and writes it to its slot from there, so the host reads run
// under the attention's own work.
static hipError_t enqueue_attention(const ess_dims& d, const ess_layer_io& io,
                                    hipStream_t st) {
  const ess::TailView tail{io.tail_rows, io.tail_rows ? io.tail_start : nullptr,
                          io.tail_rows ? io.tail_block : 1};
  return ess::launch_sparse_mla(d, io.q_abs, io.sel_pos, io.sel_slot,
                                io.row_dst, io.n_sel, io.pool,
                                io.host_entries ? nullptr : io.host_view,
                                io.out, io.lse, io.ws, st, 0, io.host_entries,
                                tail);
}

ess_status ess_decode_step(const ess_dims* d, int32_t n_layers,
                           const ess_layer_io* layers, const int32_t* n_vis,
                           int32_t mode, hipStream_t stream,
                           hipStream_t side) {
  const char* fn = "ess_decode_step";
  ess_status s = check_dims(d, fn);
  if (s != ESS_OK) return s;
  if (n_layers < 1) return fail(ESS_ERR_INVALID, "%s: n_layers < 1", fn);
  ESS_NONNULL(layers);
  ESS_NONNULL(n_vis);
  if (mode != ESS_MODE_FILL && mode != ESS_MODE_INLINE &&
      mode != ESS_MODE_PREFETCH)
    return fail(ESS_ERR_INVALID, "%s: unknown mode %d", fn, mode);
  if ((s = check_indexer(d, fn)) != ESS_OK) return s;
  if (mode == ESS_MODE_FILL) {
    if ((s = check_update(d, d->pool_slots, 1, fn)) != ESS_OK) return s;
  } else {
    if ((s = check_update(d, d->topk, d->mtp, fn)) != ESS_OK) return s;
    if ((s = check_mla(d, fn)) != ESS_OK) return s;
  }
  if (mode == ESS_MODE_PREFETCH && (side == stream))
    return fail(ESS_ERR_INVALID, "%s: prefetch needs a second stream", fn);
  const size_t ws_need = ws_total(*d);
  // The top-k and position-list regions of a layer's workspace (the first
  // fill uses them only when the layer brings a full workspace; it is not
  // required there).
  auto tws = [&](const ess_layer_io& io) -> void* {
    if (!io.ws || io.ws_bytes < ws_need || topk_region(*d) == 0) return nullptr;
    return static_cast<char*>(io.ws) + attn_region(*d);
  };
  auto lws = [&](const ess_layer_io& io) -> void* {
    if (!io.ws || io.ws_bytes < ws_need) return nullptr;
    return static_cast<char*>(io.ws) + attn_region(*d) + topk_region(*d);
  };
  for (int l = 0; l < n_layers; ++l) {
    if ((s = check_layer(layers[l], mode, l)) != ESS_OK) return s;
    if (mode != ESS_MODE_FILL && layers[l].ws_bytes < ws_need)
      return fail(ESS_ERR_NOMEM, "%s: layer %d workspace of %zu bytes, need %zu",
                  fn, l, layers[l].ws_bytes, ws_need);
  }

  hipError_t e = hipSuccess;
  if (mode == ESS_MODE_FILL) {
    const int C = d->pool_slots;
    for (int l = 0; l < n_layers && e == hipSuccess; ++l) {
      const ess_layer_io& io = layers[l];
      e = enqueue_select(*d, io, n_vis, C, 1, tws(io), lws(io), stream);
      if (e == hipSuccess)
        e = io.host_entries
                ? ess::launch_entry_copy(*d, C, io.miss_pos, io.miss_slot,
                                         io.n_miss, io.host_entries, io.pool,
                                         stream)
                : ess::launch_miss_copy(*d, C, io.miss_pos, io.miss_slot,
                                        io.n_miss, io.host_view, io.pool,
                                        stream);
    }
    return e == hipSuccess ? ESS_OK : hip_fail(e, fn);
  }
  if (mode == ESS_MODE_INLINE) {
    for (int l = 0; l < n_layers && e == hipSuccess; ++l) {
      const ess_layer_io& io = layers[l];
      e = enqueue_select(*d, io, n_vis, d->topk, d->mtp, tws(io), lws(io), stream);
      if (e == hipSuccess) e = enqueue_attention(*d, io, stream);
    }
    return e == hipSuccess ? ESS_OK : hip_fail(e, fn);
  }

  // Prefetch: the side stream selects every layer (scores, top-k, pool
  // update) back to back, running ahead; the main stream runs layer l's
  // gather + attention once layer l is selected.  Layer l+1's selection thus
  // runs under layer l's miss transfer and attention, and the host link
  // carries the layers' misses nearly back to back.  (Measured on MI355X: a
  // miss copy kernel beside an attention slows both, so the transfer and
  // the attention stay on one stream.)
  hipEvent_t* ev;
  if ((s = get_events((size_t)n_layers + 1, &ev)) != ESS_OK) return s;
  e = hipEventRecord(ev[n_layers], stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(side, ev[n_layers], 0);
  for (int l = 0; l < n_layers && e == hipSuccess; ++l) {
    // Layer 0's selection runs alone (the side stream waited for the main
    // stream's earlier work); later layers' run beside an attention.
    e = enqueue_select(*d, layers[l], n_vis, d->topk, d->mtp, tws(layers[l]), lws(layers[l]),
                       side, l > 0);
    if (e == hipSuccess) e = hipEventRecord(ev[l], side);
  }
  for (int l = 0; l < n_layers && e == hipSuccess; ++l) {
    const ess_layer_io& io = layers[l];
    e = hipStreamWaitEvent(stream, ev[l], 0);
    if (e == hipSuccess) e = enqueue_attention(*d, io, stream);
  }
  return e == hipSuccess ? ESS_OK : hip_fail(e, fn);
}

ess_status ess_tail_init(ess_tail* t, const ess_dims* d, uint16_t* rows,
                         uint8_t* entries, int32_t block, const int32_t* n_ctx,
                         int32_t* state_dev, hipStream_t stream) {
  const char* fn = "ess_tail_init";
  ESS_NONNULL(t);
  t->rows = nullptr;
  t->entries = nullptr;
  t->host = nullptr;
  t->events = nullptr;
  ess_status s = check_dims(d, fn);
  if (s != ESS_OK) return s;
  ESS_NONNULL(rows);
  ESS_NONNULL(n_ctx);
  ESS_NONNULL(state_dev);
  const int B = d->batch;
  if (block < 1) return fail(ESS_ERR_INVALID, "%s: block must be >= 1", fn);
  if (entries && (reinterpret_cast<uintptr_t>(entries) & 15))
    return fail(ESS_ERR_INVALID, "%s: entries must be 16-byte aligned", fn);
  for (int b = 0; b < B; ++b)
    if (n_ctx[b] < 1 || n_ctx[b] > d->ctx_len)
      return fail(ESS_ERR_INVALID, "%s: n_ctx[%d] = %d outside [1, ctx_len]", fn, b,
                  n_ctx[b]);
  int32_t* host = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * 3 * B));
  void** events = static_cast<void**>(std::calloc(2 * (size_t)B, sizeof(void*)));
  if (!host || !events) {
    std::free(host);
    std::free(events);
    return fail(ESS_ERR_NOMEM, "%s: host allocation failed", fn);
  }
  for (int b = 0; b < B; ++b) host[b] = host[B + b] = host[2 * B + b] = n_ctx[b];
  t->rows = rows;
  t->entries = entries;
  t->block = block;
  t->batch = B;
  t->host = host;
  t->state_dev = state_dev;
  t->events = events;
  hipError_t e = hipSuccess;
  for (int i = 0; i < 2 * B && e == hipSuccess; ++i) {
    hipEvent_t ev;
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e == hipSuccess) events[i] = ev;
  }
  // The device copy of (first, n_ctx, start): the append kernel advances it,
  // the attention reads start.  Copied from the library's host array, which
  // stays alive until ess_tail_release, after a wait for the copy.
  if (e == hipSuccess)
    e = hipMemcpyAsync(state_dev, host, sizeof(int32_t) * 3 * B,
                       hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    ess_tail_release(t);
    return hip_fail(e, fn);
  }
  return ESS_OK;
}

ess_status ess_tail_release(ess_tail* t) {
  if (!t) return ESS_OK;
  if (t->events)
    for (int i = 0; i < 2 * t->batch; ++i)
      if (t->events[i]) (void)hipEventDestroy(static_cast<hipEvent_t>(t->events[i]));
  std::free(t->events);
  std::free(t->host);
  t->events = nullptr;
  t->host = nullptr;
  t->rows = nullptr;
  t->entries = nullptr;
  return ESS_OK;
}

ess_status ess_append_tokens(const ess_dims* d, ess_tail* t,
                             const uint8_t* new_keys, const uint16_t* new_lat,
                             uint8_t* k_idx, int32_t* n_vis, void* host_store,
                             hipStream_t stream, hipStream_t d2h) {
  const char* fn = "ess_append_tokens";
  ess_status s = check_dims(d, fn);
  if (s != ESS_OK) return s;
  if ((s = check_indexer(d, fn)) != ESS_OK) return s;
  ESS_NONNULL(t);
  ESS_NONNULL(new_keys);
  ESS_NONNULL(new_lat);
  ESS_NONNULL(k_idx);
  ESS_NONNULL(n_vis);
  ESS_NONNULL(host_store);
  if (!t->rows || !t->host || !t->events || !t->state_dev)
    return fail(ESS_ERR_INVALID, "%s: tail is not initialised (ess_tail_init)", fn);
  if (t->batch != d->batch)
    return fail(ESS_ERR_INVALID, "%s: tail of %d requests, dims of %d", fn,
                t->batch, d->batch);
  if (stream == d2h)
    return fail(ESS_ERR_INVALID, "%s: the write-back needs a stream of its own", fn);
  const int m = d->mtp, B = d->batch, L = d->ctx_len, blk = t->block;
  if (blk < m)
    return fail(ESS_ERR_UNSUPPORTED, "%s: tail block of %d tokens < mtp %d", fn, blk, m);
  int32_t* first = t->host;
  int32_t* ctx = t->host + B;
  int32_t* start = t->host + 2 * B;
  for (int b = 0; b < B; ++b)
    if (ctx[b] + m > L)
      return fail(ESS_ERR_INVALID, "%s: request %d: context of %d + %d tokens exceeds ctx_len %d",
                  fn, b, ctx[b], m, L);
  hipEvent_t* ev;
  if ((s = get_events(1, &ev)) != ESS_OK) return s;
  hipError_t e = hipSuccess;
  // A block's buffer last held the block two before it: that block's
  // write-back must finish before its rows are overwritten.
  for (int b = 0; b < B && e == hipSuccess; ++b) {
    const int n0 = ctx[b], n1 = n0 + m;
    for (int c = n0 / blk; c <= (n1 - 1) / blk && e == hipSuccess; ++c)
      if (c * blk >= n0 && c >= 2 && (c - 1) * blk - 1 >= first[b])
        e = hipStreamWaitEvent(stream, static_cast<hipEvent_t>(t->events[2 * b + (c & 1)]), 0);
  }
  if (e == hipSuccess)
    e = ess::launch_append_tokens(*d, blk, new_keys, new_lat, k_idx, t->rows,
                                  t->entries, n_vis, t->state_dev, stream);
  // Blocks filled by this append go back to the host store on d2h.
  bool recorded = false;
  for (int b = 0; b < B && e == hipSuccess; ++b) {
    const int n0 = ctx[b], n1 = n0 + m;
    for (int c = n0 / blk; c <= (n1 - 1) / blk && e == hipSuccess; ++c) {
      const int last = (c + 1) * blk - 1;
      if (last < n0 || last >= n1) continue;
      if (!recorded) {
        e = hipEventRecord(ev[0], stream);
        if (e == hipSuccess) e = hipStreamWaitEvent(d2h, ev[0], 0);
        recorded = true;
        if (e != hipSuccess) break;
      }
      // Rows of the block as the host store holds them: bf16 rows, or the
      // entries quantized at append.
      const int p0 = std::max(first[b], c * blk);
      const size_t unit = t->entries ? ess::kEntryBytes : ess::kLat * sizeof(uint16_t);
      const char* src = t->entries ? reinterpret_cast<const char*>(t->entries)
                                   : reinterpret_cast<const char*>(t->rows);
      e = hipMemcpyAsync(static_cast<char*>(host_store) + ((size_t)b * L + p0) * unit,
                         src + ((size_t)b * 2 * blk + (c & 1) * blk + p0 % blk) * unit,
                         (size_t)(last + 1 - p0) * unit, hipMemcpyDeviceToHost, d2h);
      if (e == hipSuccess)
        e = hipEventRecord(static_cast<hipEvent_t>(t->events[2 * b + (c & 1)]), d2h);
    }
  }
  if (e != hipSuccess) return hip_fail(e, fn);
  for (int b = 0; b < B; ++b) {
    ctx[b] += m;
    start[b] = std::max(first[b], ((ctx[b] - 1) / blk - 1) * blk);
  }
  return ESS_OK;
}

size_t ess_prefill_ws_bytes(int32_t rows) {
  return rows < 1 ? 0 : ess::prefill_ws_bytes(rows);
}

ess_status ess_prefill_layers(int32_t n_layers, int32_t rows, int32_t n_hist,
                              int32_t n_new, uint16_t* host_kv,
                              const uint16_t* new_kv, uint16_t* bufs,
                              float* layer_out, void* ws, size_t ws_bytes,
                              const int32_t* onload_layer_map,
                              int32_t* binding, int32_t compute_reps,
                              int32_t load_layer0, hipStream_t compute,
                              hipStream_t h2d, hipStream_t d2h) {
  const char* fn = "ess_prefill_layers";
  if (n_layers < 1 || rows < 1 || n_hist < 0 || n_new < 0 ||
      n_hist + n_new < 1 || n_hist + n_new > rows || compute_reps < 1)
    return fail(ESS_ERR_INVALID,
                "%s: bad sizes (n_layers %d, rows %d, n_hist %d, n_new %d, reps %d)",
                fn, n_layers, rows, n_hist, n_new, compute_reps);
  ESS_NONNULL(host_kv);
  ESS_NONNULL(bufs);
  ESS_NONNULL(layer_out);
  ESS_NONNULL(ws);
  if (n_new > 0) ESS_NONNULL(new_kv);
  if (compute == h2d || compute == d2h || h2d == d2h)
    return fail(ESS_ERR_INVALID, "%s: compute, h2d and d2h must be three streams", fn);
  const size_t need = ess::prefill_ws_bytes(rows);
  if (ws_bytes < need)
    return fail(ESS_ERR_NOMEM, "%s: workspace of %zu bytes, need %zu", fn,
                ws_bytes, need);

  // Bindings (checked before anything is enqueued): layers 1..3 take B1..B3;
  // layer i >= 1 releases its buffer after its compute and write-back, and
  // its scheduling point binds the oldest released buffer to the map's
  // layer.
  constexpr int kBufs = 4;
  std::vector<int> bind(n_layers, -1), freed_by(n_layers, -1), trigger(n_layers, -1);
  std::vector<std::pair<int, int>> freeq;        // (buffer, released by layer)
  bind[0] = 0;
  for (int b = 1; b < kBufs; ++b) freeq.emplace_back(b, -1);
  for (int l = 1; l < kBufs && l < n_layers; ++l) {
    bind[l] = freeq.front().first;
    freed_by[l] = freeq.front().second;
    freeq.erase(freeq.begin());
  }
  for (int i = 0; i < n_layers; ++i) {
    if (bind[i] < 0)
      return fail(ESS_ERR_INVALID, "%s: layer %d is not loaded when its turn comes", fn, i);
    if (i == 0) continue;
    freeq.emplace_back(bind[i], i);
    int j;
    if (!onload_layer_map) {
      j = i + kBufs - 1;
      if (j >= n_layers) continue;
    } else {
      j = onload_layer_map[i];
      if (j < 0) continue;
    }
    if (j <= i || j >= n_layers || bind[j] >= 0)
      return fail(ESS_ERR_INVALID,
                  "%s: onload_layer_map[%d] = %d is not a future, unloaded layer", fn, i, j);
    bind[j] = freeq.front().first;
    freed_by[j] = freeq.front().second;
    trigger[j] = i;
    freeq.erase(freeq.begin());
  }
  if (binding)
    for (int l = 0; l < n_layers; ++l) binding[l] = bind[l];

  // Events: per layer loaded (h2d), computed (compute), released (d2h).
  hipEvent_t* ev;
  ess_status st;
  if ((st = get_events(3 * (size_t)n_layers + 1, &ev)) != ESS_OK) return st;
  hipEvent_t* loaded = ev;
  hipEvent_t* computed = ev + n_layers;
  hipEvent_t* released = ev + 2 * (size_t)n_layers;
  hipEvent_t start = ev[3 * (size_t)n_layers];
  const size_t row_b = (size_t)ess::kLat * sizeof(uint16_t);
  const size_t layer_rows = (size_t)rows * ess::kLat;
  auto host_layer = [&](int l) { return host_kv + (size_t)l * layer_rows; };
  auto buf_of = [&](int l) { return bufs + (size_t)bind[l] * layer_rows; };
  float* part = static_cast<float*>(ws);

  hipError_t e = hipEventRecord(start, compute);
  if (e == hipSuccess) e = hipStreamWaitEvent(h2d, start, 0);
  if (e == hipSuccess) e = hipStreamWaitEvent(d2h, start, 0);
  auto load = [&](int l) -> hipError_t {
    hipError_t r = hipSuccess;
    if (n_hist > 0)
      r = hipMemcpyAsync(buf_of(l), host_layer(l), (size_t)n_hist * row_b,
                         hipMemcpyHostToDevice, h2d);
    if (r == hipSuccess) r = hipEventRecord(loaded[l], h2d);
    return r;
  };
  if (e == hipSuccess && load_layer0) e = load(0);
  for (int l = 1; l < n_layers && e == hipSuccess; ++l)
    if (trigger[l] < 0) e = load(l);
  for (int i = 0; i < n_layers && e == hipSuccess; ++i) {
    if (i > 0 || load_layer0) e = hipStreamWaitEvent(compute, loaded[i], 0);
    if (e == hipSuccess)
      e = ess::launch_prefill_compute(n_new ? new_kv + (size_t)i * n_new * ess::kLat : nullptr,
                                      n_new, buf_of(i), n_hist, compute_reps, part,
                                      layer_out + (size_t)i * ess::kLat, compute);
    if (e == hipSuccess) e = hipEventRecord(computed[i], compute);
    if (e == hipSuccess) e = hipStreamWaitEvent(d2h, computed[i], 0);
    if (e == hipSuccess && n_new > 0)
      e = hipMemcpyAsync(host_layer(i) + (size_t)n_hist * ess::kLat,
                         buf_of(i) + (size_t)n_hist * ess::kLat,
                         (size_t)n_new * row_b, hipMemcpyDeviceToHost, d2h);
    if (e == hipSuccess) e = hipEventRecord(released[i], d2h);
    // Loads issued at this layer's scheduling point.
    for (int j = i + 1; j < n_layers && e == hipSuccess; ++j) {
      if (trigger[j] != i) continue;
      e = hipStreamWaitEvent(h2d, released[freed_by[j]], 0);
      if (e == hipSuccess && freed_by[j] != i) e = hipStreamWaitEvent(h2d, computed[i], 0);
      if (e == hipSuccess) e = load(j);
    }
  }
  // Every write-back done before later work on the compute stream.
  if (e == hipSuccess) e = hipStreamWaitEvent(compute, released[n_layers - 1], 0);
  return e == hipSuccess ? ESS_OK : hip_fail(e, fn);
}

ess_status ess_host_alloc(size_t bytes, void** host_ptr, void** dev_view) {
  const char* fn = "ess_host_alloc";
  ESS_NONNULL(host_ptr);
  ESS_NONNULL(dev_view);
  if (bytes == 0) return fail(ESS_ERR_INVALID, "%s: zero bytes", fn);
  void* p = nullptr;
  hipError_t e = hipHostMalloc(&p, bytes,
                               hipHostMallocMapped | hipHostMallocNonCoherent);
  if (e != hipSuccess || !p)
    return fail(ESS_ERR_NOMEM, "%s: hipHostMalloc(%zu): %s", fn, bytes,
                hipGetErrorString(e));
  void* dv = nullptr;
  e = hipHostGetDevicePointer(&dv, p, 0);
  if (e != hipSuccess) {
    (void)hipHostFree(p);
    return hip_fail(e, "hipHostGetDevicePointer");
  }
  *host_ptr = p;
  *dev_view = dv;
  return ESS_OK;
}

ess_status ess_host_free(void* host_ptr) {
  if (!host_ptr) return ESS_OK;
  hipError_t e = hipHostFree(host_ptr);
  return e == hipSuccess ? ESS_OK : hip_fail(e, "hipHostFree");
}

const char* ess_status_string(ess_status s) {
  switch (s) {
    case ESS_OK: return "ok";
    case ESS_ERR_INVALID: return "invalid argument";
    case ESS_ERR_UNSUPPORTED: return "unsupported shape";
    case ESS_ERR_CAPACITY: return "pool capacity exceeded";
    case ESS_ERR_HIP: return "HIP runtime error";
    case ESS_ERR_NOMEM: return "out of memory";
  }
  return "unknown status";
}

const char* ess_last_error(void) { return g_err.c_str(); }

}  // extern "C"
