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
// One 1024-thread workgroup per request.
#include "block_util.h"
#include "ess_internal.h"

namespace ess {
namespace {

constexpr int NT = 1024;

struct Ring {
  int32_t slot;
  int32_t stamp;
};

__device__ __forceinline__ LruHeader* hdr_of(void* lru, size_t stride, int b) {
  return reinterpret_cast<LruHeader*>(static_cast<char*>(lru) + stride * b);
}

__global__ __launch_bounds__(NT) void pool_reset_kernel(
    int32_t* __restrict__ cache_slots, int32_t* __restrict__ slot_pos,
    void* lru, size_t stride, int L, int C) {
  const int b = blockIdx.y;
  LruHeader* h = hdr_of(lru, stride, b);
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
  }
}

// Entry key: (position * n_tok + token) << 32 | row; ascending order gives
// positions ascending and, for a repeated position, the smallest token first.
__global__ __launch_bounds__(NT) void pool_update_kernel(
    const int32_t* __restrict__ sel_pos, const int32_t* __restrict__ n_sel,
    int32_t* __restrict__ cache_slots, int32_t* __restrict__ slot_pos,
    void* lru, size_t stride, int32_t* __restrict__ miss_pos,
    int32_t* __restrict__ miss_slot, int32_t* __restrict__ n_miss_out,
    int32_t* __restrict__ n_evict_out, int32_t* __restrict__ row_dst,
    int32_t* __restrict__ sel_slot_post, int L, int C, int k, int n_tok,
    int epow2) {
  extern __shared__ uint64_t ent[];            // epow2 entries
  __shared__ uint32_t tmp[NT / 64 + 1];
  __shared__ int s_head_new;

  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  LruHeader* h = hdr_of(lru, stride, b);
  int32_t* stamp = reinterpret_cast<int32_t*>(h + 1);
  Ring* ring = reinterpret_cast<Ring*>(stamp + C);
  int32_t* cs = cache_slots + (size_t)b * L;
  int32_t* sp = slot_pos + (size_t)b * C;
  const size_t list0 = (size_t)b * n_tok * k;   // copy-list base
  const size_t rows0 = (size_t)b * n_tok * k;   // per-row arrays base

  const int head0 = h->head, tail0 = h->tail, free_head = h->free_head;
  const int epoch = h->epoch, cap = h->cap;

  int off[5];
  off[0] = 0;
  for (int j = 0; j < n_tok; ++j)
    off[j + 1] = off[j] + min(max(n_sel[b * n_tok + j], 0), k);
  const int n_e = off[n_tok];

  // 0. Row outputs start empty.
  for (int i = tid; i < n_tok * k; i += NT) {
    row_dst[rows0 + i] = -1;
    sel_slot_post[rows0 + i] = -1;
  }
  // 1. Entries of every way, then sort.
  for (int e = tid; e < epow2; e += NT) {
    uint64_t key = ~0ull;
    if (e < n_e) {
      int j = 0;
      while (e >= off[j + 1]) ++j;
      const int i = e - off[j];
      const int pos = sel_pos[rows0 + (size_t)j * k + i];
      if (pos >= 0 && pos < L)   // out-of-range positions are dropped
        key = ((uint64_t)((uint32_t)pos * (uint32_t)n_tok + j) << 32) | (uint32_t)i;
      else
        h->err = 2;
    }
    ent[e] = key;
  }
  __syncthreads();
  bitonic_sort_u64<NT, false>(ent, epow2);

  // 2. Unique positions (first entry of each run) and their lookup.  Dropped
  // entries sort last (key ~0) and end the run.
  const int per = (epow2 + NT - 1) / NT;       // entries per thread, contiguous
  const int e0 = tid * per;
  auto first_of_run = [&](int e, uint32_t pk) {
    return e == 0 || (uint32_t)(ent[e - 1] >> 32) / n_tok != pk / n_tok;
  };
  uint32_t n_u_mine = 0, n_m_mine = 0;
  for (int q = 0; q < per; ++q) {
    const int e = e0 + q;
    if (e >= n_e) break;
    if (ent[e] == ~0ull) break;
    const uint32_t pk = (uint32_t)(ent[e] >> 32);
    if (first_of_run(e, pk)) {
      ++n_u_mine;
      const int slot = cs[pk / n_tok];
      if (slot < 0 || slot >= C) ++n_m_mine;
      else stamp[slot] = epoch;                // touched: old ring entry dies
    }
  }
  uint32_t n_u, n_miss;
  const uint32_t u_base = block_exscan<NT>(n_u_mine, tmp, &n_u);
  const uint32_t m_base = block_exscan<NT>(n_m_mine, tmp, &n_miss);

  // 3. Victims: never-used slots first, then the ring from its head.
  const int n_free = C - free_head;
  const int use_free = min((int)n_miss, n_free);
  const int n_ev = (int)n_miss - use_free;
  int head = head0;
  int found = 0;
  if (n_ev > 0) {
    if (tid == 0) s_head_new = head0;
    while (found < n_ev) {
      const int idx = head + tid;
      bool live = false;
      int slot = -1;
      if (idx < tail0) {
        const Ring r = ring[idx];
        slot = r.slot;
        live = slot >= 0 && slot < C && stamp[slot] == r.stamp;
      }
      uint32_t tot;
      const uint32_t rank = block_exscan<NT>(live ? 1u : 0u, tmp, &tot);
      if (live && found + (int)rank < n_ev) {
        const int v = found + (int)rank;
        miss_slot[list0 + use_free + v] = slot;
        const int old = sp[slot];
        if (old >= 0 && old < L) cs[old] = -1;   // evict
        if (v == n_ev - 1) s_head_new = idx + 1;
      }
      __syncthreads();
      if (found + (int)tot >= n_ev) {
        head = s_head_new;
        found = n_ev;
      } else {
        found += (int)tot;
        head += NT;
        if (head >= tail0) {                   // ran dry: inconsistent state
          if (tid == 0) h->err = 1;
          break;
        }
      }
    }
  }
  __syncthreads();

  // 4. Pair misses (ascending position) with victims (in victim order).  A
  // ring that ran dry (inconsistent state, flagged above) leaves the misses
  // past the victims found unpaired.
  {
    const int paired = use_free + found;
    uint32_t mi = m_base;
    for (int q = 0; q < per; ++q) {
      const int e = e0 + q;
      if (e >= n_e) break;
      const uint64_t key = ent[e];
      if (key == ~0ull) break;
      const uint32_t pk = (uint32_t)(key >> 32);
      if (!first_of_run(e, pk)) continue;
      const int pos = (int)(pk / n_tok);
      const int cur = cs[pos];
      if (cur >= 0 && cur < C) continue;       // hit (evictions never hit U)
      const int v = (int)mi < use_free ? free_head + (int)mi
                                       : miss_slot[list0 + mi];
      if ((int)mi < paired && v >= 0 && v < C) {
        cs[pos] = v;
        sp[v] = pos;
        stamp[v] = epoch;
        miss_pos[list0 + mi] = pos;
        miss_slot[list0 + mi] = v;
        const int j = (int)(pk % n_tok);
        const int i = (int)(uint32_t)key;
        row_dst[rows0 + (size_t)j * k + i] = v;  // smallest token's row
      }
      ++mi;
    }
  }
  __syncthreads();

  // 5. Make room on the ring: compact live entries to the front in order.
  int tail = tail0;
  if (tail + (int)n_u > cap) {
    int dst = 0;
    for (int src = head; src < tail; src += NT) {
      const int idx = src + tid;
      Ring r = {0, 0};
      bool live = false;
      if (idx < tail) {
        r = ring[idx];
        live = r.slot >= 0 && r.slot < C && stamp[r.slot] == r.stamp;
      }
      uint32_t tot;
      const uint32_t rank = block_exscan<NT>(live ? 1u : 0u, tmp, &tot);
      if (live) ring[dst + rank] = r;
      dst += (int)tot;
      __syncthreads();
    }
    head = 0;
    tail = dst;
  }

  // 6. Push the union in ascending position order with current slots.
  for (int q = 0, u = (int)u_base; q < per; ++q) {
    const int e = e0 + q;
    if (e >= n_e) break;
    if (ent[e] == ~0ull) break;
    const uint32_t pk = (uint32_t)(ent[e] >> 32);
    if (!first_of_run(e, pk)) continue;
    Ring r;
    r.slot = cs[pk / n_tok];
    r.stamp = epoch;
    ring[tail + u] = r;
    ++u;
  }
  __syncthreads();

  // 7. Slots after the update for every selected row.
  for (int i = tid; i < n_tok * k; i += NT) {
    const int j = i / k, r = i % k;
    if (r < min(n_sel[b * n_tok + j], k)) {
      const int pos = sel_pos[rows0 + i];
      if (pos >= 0 && pos < L) sel_slot_post[rows0 + i] = cs[pos];
    }
  }
  if (tid == 0) {
    h->head = head;
    h->tail = tail + (int)n_u;
    h->free_head = free_head + use_free;
    h->epoch = epoch + 1;
    n_miss_out[b] = (int)n_miss;
    n_evict_out[b] = n_ev;
  }
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

hipError_t launch_pool_update(const ess_dims& d, int k, int n_tok,
                              const int32_t* sel_pos, const int32_t* n_sel,
                              int32_t* cache_slots, int32_t* slot_pos,
                              void* lru, int32_t* miss_pos,
                              int32_t* miss_slot, int32_t* n_miss,
                              int32_t* n_evict, int32_t* row_dst,
                              int32_t* sel_slot_post, hipStream_t s) {
  const size_t stride = lru_bytes_per_req(d.pool_slots);
  const int epow2 = pow2_at_least(n_tok * k);
  const size_t lds = (size_t)epow2 * sizeof(uint64_t);
  hipError_t e = hipFuncSetAttribute((const void*)pool_update_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)(kMaxTopk * sizeof(uint64_t)));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pool_update_kernel, dim3(d.batch), dim3(NT), lds, s,
                     sel_pos, n_sel, cache_slots, slot_pos, lru, stride,
                     miss_pos, miss_slot, n_miss, n_evict, row_dst,
                     sel_slot_post, d.ctx_len, d.pool_slots, k, n_tok, epow2);
  return hipGetLastError();
}

}  // namespace ess
