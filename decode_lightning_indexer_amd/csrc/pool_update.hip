// Residency update of the hot latent pool, O(m*k) per request and step.
//
// The pages keep a per-request int32 reverse index cache_slots (position ->
// slot, -1 if absent) so that a lookup is O(1) and managing the pool costs
// O(k) + O(#misses) instead of a scan of the pool (FlashOffloading analysis,
// section "cache_slots").  One steady-state step takes the union of the MTP
// ways, finds the misses, picks as many victims from the pool minus the
// union, pairs misses with victims one to one and rewrites cache_slots, so
// the pool size never changes (same page, "five steps and the MTP union").
// ESS keeps the hot subset with LRU (ESS concept page, "core mechanism").
//
// LRU order without a scan of the pool: every update pushes the (slot,
// stamp) of each union member, in ascending position order, onto a
// per-request ring; the slot's current stamp lives in slot_stamp.  A ring
// entry is live iff its stamp equals the slot's stamp, so the ring read from
// its head, skipping dead entries, lists the resident slots from least to
// most recently used - (last update in a union, position) order.  Hits are
// re-stamped before the victim scan, so union members are never victims.
// Every entry is read at most once by the head, so the cost is amortised
// O(|union|) per update.  When the ring would overflow, its live entries
// (at most C) are compacted to the front in order.
//
#include "pool_update_body.h"

namespace ess {
namespace {

using pool::NT;
using pool::kTwoBufferMax;

__global__ __launch_bounds__(NT) void pool_reset_kernel(
    int32_t* __restrict__ cache_slots, int32_t* __restrict__ slot_pos,
    void* lru, size_t stride, int L, int C) {
  const int b = blockIdx.y;
  LruHeader* h = pool::hdr_of(lru, stride, b);
  int32_t* stamp = reinterpret_cast<int32_t*>(h + 1);
  const int i0 = blockIdx.x * NT + threadIdx.x;
  for (int i = i0; i < L; i += gridDim.x * NT) cache_slots[(size_t)b * L + i] = -1;
  for (int i = i0; i < C; i += gridDim.x * NT) {
    slot_pos[(size_t)b * C + i] = -1;
    stamp[i] = -1;
  }
  if (i0 == 0) {
    h->head = 0;
    h->tail = 0;
    h->free_head = 0;
    h->epoch = 0;
    h->cap = lru_ring_cap(C);
    h->err = 0;
    h->compactions = 0;
    h->pad = 0;
  }
}

__global__ void pool_status_kernel(const void* lru, size_t stride, int B,
                                   int32_t* __restrict__ status) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const LruHeader* h = reinterpret_cast<const LruHeader*>(
      static_cast<const char*>(lru) + stride * b);
  status[4 * b + 0] = h->err;
  status[4 * b + 1] = h->compactions;
  status[4 * b + 2] = h->epoch;
  status[4 * b + 3] = h->tail - h->head;
}

// One 1024-thread workgroup per request.  MERGE: the selections come as
// position-ordered lists per token and are merged, not sorted.
template <bool MERGE>
__global__ __launch_bounds__(NT) void pool_update_kernel(pool::Args a) {
  extern __shared__ uint64_t smem_ent[];       // epow2 entries (x2: sort target)
  pool::update_request<false, false, MERGE>(a, blockIdx.x, smem_ent, nullptr, nullptr, 0);
}

}  // namespace

hipError_t launch_pool_reset(const ess_dims& d, int32_t* cache_slots,
                             int32_t* slot_pos, void* lru, hipStream_t s) {
  const size_t stride = lru_bytes_per_req(d.pool_slots);
  const int mx = d.ctx_len > d.pool_slots ? d.ctx_len : d.pool_slots;
  int gx = (mx + NT - 1) / NT;
  if (gx > 64) gx = 64;
  hipLaunchKernelGGL(pool_reset_kernel, dim3(gx, d.batch), dim3(NT), 0, s,
                     cache_slots, slot_pos, lru, stride, d.ctx_len,
                     d.pool_slots);
  return hipGetLastError();
}

hipError_t launch_pool_status(const ess_dims& d, const void* lru,
                              int32_t* status, hipStream_t s) {
  const size_t stride = lru_bytes_per_req(d.pool_slots);
  hipLaunchKernelGGL(pool_status_kernel, dim3((d.batch + 255) / 256), dim3(256), 0,
                     s, lru, stride, d.batch, status);
  return hipGetLastError();
}

hipError_t launch_pool_update(const ess_dims& d, int k, int n_tok,
                              const int32_t* sel_pos, const int32_t* n_sel,
                              int32_t* cache_slots, int32_t* slot_pos,
                              void* lru, int32_t* miss_pos,
                              int32_t* miss_slot, int32_t* n_miss,
                              int32_t* n_evict, int32_t* row_dst,
                              int32_t* sel_slot_post, hipStream_t s,
                              const int32_t* sel_slot_pre, PosLists lists) {
  const size_t stride = lru_bytes_per_req(d.pool_slots);
  // The sort buffer holds at least one entry per thread.
  const int epow2 = pow2_at_least(n_tok * k) < NT ? NT : pow2_at_least(n_tok * k);
  const int two = epow2 <= kTwoBufferMax ? 1 : 0;
  const size_t lds = (size_t)epow2 * sizeof(uint64_t) * (two ? 2 : 1);
  int bits = 0;
  while ((1 << bits) < d.ctx_len) ++bits;
  const int pos_shift = bits > 11 ? bits - 11 : 0;
  // Position-ordered lists are merged in place of the sort (the lists'
  // positions take the second buffer).
  const bool merge = lists.pos != nullptr && two;
  const void* fn = merge ? (const void*)pool_update_kernel<true>
                         : (const void*)pool_update_kernel<false>;
  hipError_t e = ensure_dyn_lds(fn, (int)(kMaxTopk * sizeof(uint64_t)));
  if (e != hipSuccess) return e;
  const pool::Args a{sel_pos, n_sel, cache_slots, slot_pos, lru, stride,
                     miss_pos, miss_slot, n_miss, n_evict, row_dst,
                     sel_slot_post, d.ctx_len, d.pool_slots, k, n_tok, epow2,
                     two, pos_shift, sel_slot_pre,
                     merge ? lists : PosLists{nullptr, nullptr, nullptr}};
  if (merge)
    hipLaunchKernelGGL(pool_update_kernel<true>, dim3(d.batch), dim3(NT), lds, s, a);
  else
    hipLaunchKernelGGL(pool_update_kernel<false>, dim3(d.batch), dim3(NT), lds, s, a);
  return hipGetLastError();
}

}  // namespace ess
