// Top-k selection per (request, query token) with the residency lookup read
// off the winners.
//
// The pages fold the cache_slots lookup into the top-k itself by packing the
// candidate's index and slot with its score into one int32 selection key
// (FlashOffloading analysis, section "LIM: packing the index into the
// score") and note that this caps sequence length and pool size.  At 1M
// positions and 16K slots the pieces do not fit in 32 bits, so here the key
// is 64 bits - the order-preserving score bits above the complemented
// position (equal scores: lower position wins) - and the slot of each winner
// is gathered in the same final pass that writes the winners.
//
// One 1024-thread workgroup per row (the rows are few: B * m); scores are
// read with 16-byte loads, all of a thread's loads for a chunk in flight
// together:
//   1. min and max of the order-preserving keys of the visible positions;
//   2. radix passes of up to 11 bits starting at the highest bit where min
//      and max differ, each narrowing the bin that holds the k-th key, until
//      that bin holds at most one wave's worth of keys or the bits run out;
//   3. keys above the bin are winners: a histogram of them over 2048 buckets
//      of equal score width, a scan, and a scatter into LDS grouped by
//      bucket.  Keys in the bin are candidates: one wave sorts them and the
//      best `need` take the last ranks (a bin of equal keys too large for a
//      wave takes them in position order with workgroup scans);
//   4. each winner's rank is its bucket's start plus the number of larger
//      keys in its bucket; it is written straight to that rank of the
//      outputs with its slot.  A bucket too large for that (a long run of
//      equal or near-equal scores) falls back to a full bitonic sort.
#include "block_util.h"
#include "ess_internal.h"
#include "pool_update_body.h"

namespace ess {
namespace {

constexpr int NT = 1024;
constexpr int kBins = 2048;
constexpr int kSmall = 64;       // candidates sorted by one wave
constexpr int kMaxBucket = 256;  // larger winner buckets take the full sort
constexpr int kFusedMaxK = 4096;  // top-k + update in one workgroup up to this k

__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;          // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t full_key(uint32_t ok, int pos) {
  return ((uint64_t)ok << 32) | (uint32_t)(~(uint32_t)pos);
}

__device__ __forceinline__ bool in_fixed(uint32_t key, uint32_t prefix,
                                         int lo_fixed) {
  return ((uint64_t)key >> lo_fixed) == ((uint64_t)prefix >> lo_fixed);
}

// Keys are read in chunks of NT * 32: thread t holds positions
// base + (v * NT + t) * 4 + e for v < 8, e < 4, loaded as eight 16-byte
// loads issued together.  A row of at most one chunk is loaded once and kept
// in registers for every pass (RES); longer rows are streamed per pass.
constexpr int VPT = 8;                 // 16-byte loads per thread per chunk
constexpr int KPT = VPT * 4;           // keys per thread per chunk
constexpr int CHUNK = NT * KPT;        // 32768 keys

// Top-k of one (request, token) row by a 1024-thread workgroup; returns the
// number selected.  grp: kpow2 winners of LDS.  FUSE: the outputs are also
// left in LDS (rpos, rslot) for the residency update that follows in the
// same workgroup.
template <bool RES, bool FUSE>
__device__ int topk_row(
    const float* __restrict__ scores, const int32_t* __restrict__ n_vis,
    const int32_t* __restrict__ cache_slots, int32_t* __restrict__ sel_pos,
    int32_t* __restrict__ sel_slot, int32_t* __restrict__ n_sel, int L, int m,
    int n_tok, int k, int kpow2, int row, uint64_t* grp, int32_t* rpos,
    int32_t* rslot) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint64_t cand[kSmall];
  __shared__ uint32_t tmp[2 * (NT / 64) + 1];
  __shared__ uint32_t s_bin_need, s_bin_cnt, s_nc;
  __shared__ int s_bin;

  const int tid = threadIdx.x;
  const int b = row / n_tok, j = row % n_tok;
  const float* srow = scores + ((size_t)b * m + j) * L;
  int n = n_vis[b * m + j];
  n = n < 0 ? 0 : (n > L ? L : n);
  const int keff = min(k, n);
  const bool vec = (L & 3) == 0;     // rows start 16-byte aligned
  int32_t* op = sel_pos + ((size_t)b * n_tok + j) * k;
  int32_t* os = sel_slot + ((size_t)b * n_tok + j) * k;
  const int32_t* cs = cache_slots + (size_t)b * L;
  for (int i = keff + tid; i < k; i += NT) {
    op[i] = -1;
    os[i] = -1;
  }
  if (tid == 0) n_sel[b * n_tok + j] = keff;
  if (keff == 0) return 0;
  // Output row r: the selection and its slot.
#define EMIT(R, POS, SLOT)                                                    \
  do {                                                                        \
    op[R] = (POS);                                                            \
    os[R] = (SLOT);                                                           \
    if (FUSE) {                                                               \
      rpos[R] = (POS);                                                        \
      rslot[R] = (SLOT);                                                      \
    }                                                                         \
  } while (0)

  // Keys of one chunk for this thread.  A chunk wholly inside the visible
  // row (the common case) takes eight unconditional 16-byte loads, all in
  // flight together; a partial chunk takes bounds-checked scalar loads.
  uint32_t kr[KPT];
#define ESS_TOPK_LOAD(BASE)                                                   \
  do {                                                                        \
    const int base_ = (BASE);                                                 \
    if (vec && base_ + CHUNK <= n) {                                          \
      float4 f_[VPT];                                                         \
      _Pragma("unroll") for (int v = 0; v < VPT; ++v)                         \
        f_[v] = *reinterpret_cast<const float4*>(srow + base_ + (v * NT + tid) * 4); \
      _Pragma("unroll") for (int v = 0; v < VPT; ++v) {                       \
        kr[4 * v + 0] = ord_key(f_[v].x);                                     \
        kr[4 * v + 1] = ord_key(f_[v].y);                                     \
        kr[4 * v + 2] = ord_key(f_[v].z);                                     \
        kr[4 * v + 3] = ord_key(f_[v].w);                                     \
      }                                                                       \
    } else {                                                                  \
      _Pragma("unroll") for (int v = 0; v < VPT; ++v)                         \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) {                       \
          const int p_ = base_ + (v * NT + tid) * 4 + e;                      \
          kr[4 * v + e] = p_ < n ? ord_key(srow[p_]) : 0u;                    \
        }                                                                     \
    }                                                                         \
  } while (0)
#define pos_of(BASE, V, E) ((BASE) + ((V) * NT + tid) * 4 + (E))
  const int nchunks = (n + CHUNK - 1) / CHUNK;

  if (RES) ESS_TOPK_LOAD(0);
  // 1. Range of the keys.
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int c = 0; c < nchunks; ++c) {
    const int base = c * CHUNK;
    if (!RES) ESS_TOPK_LOAD(base);
#pragma unroll
    for (int v = 0; v < VPT; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (pos_of(base, v, e) < n) {
          mn = min(mn, kr[4 * v + e]);
          mx = max(mx, kr[4 * v + e]);
        }
  }
  block_minmax<NT>(mn, mx, tmp);

  // Winners are the keys >= win_lo; candidates the keys in [bin_lo, win_lo),
  // of which the best `need` are taken.
  uint64_t bin_lo = 0, win_lo = 0;
  uint32_t need = 0, cnt = 0;
  if (keff < n) {
    // Bits at and above lo_fixed are common to every key in the bin that
    // holds the k-th key; `prefix` carries them.
    int lo_fixed = (mn == mx) ? 0 : 32 - __clz(mn ^ mx);
    uint32_t prefix = mn;
    need = keff;
    cnt = n;
    // 2. Radix passes until the bin is small or the bits run out.
    while (cnt > (uint32_t)kSmall && lo_fixed > 0) {
      const int hi = lo_fixed - 1;
      const int lo = hi >= 10 ? hi - 10 : 0;
      const int nb = 1 << (hi - lo + 1);
      for (int i = tid; i < kBins; i += NT) hist[i] = 0;
      __syncthreads();
      for (int c = 0; c < nchunks; ++c) {
        const int base = c * CHUNK;
        if (!RES) ESS_TOPK_LOAD(base);
#pragma unroll
        for (int v = 0; v < VPT; ++v)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t key = kr[4 * v + e];
            if (pos_of(base, v, e) < n && in_fixed(key, prefix, lo_fixed))
              atomicAdd(&hist[(key >> lo) & (nb - 1)], 1u);
          }
      }
      __syncthreads();
      // Bins in descending order: thread t owns bins nb-1-2t and nb-2-2t.
      uint32_t h0 = 0, h1 = 0;
      const int b0 = nb - 1 - 2 * tid, b1 = b0 - 1;
      if (b0 >= 0) h0 = hist[b0];
      if (b1 >= 0) h1 = hist[b1];
      uint32_t tot;
      const uint32_t above = block_exscan<NT>(h0 + h1, tmp, &tot);
      if (b0 >= 0 && above < need && need <= above + h0) {
        s_bin = b0;
        s_bin_need = need - above;
        s_bin_cnt = h0;
      }
      if (b1 >= 0 && above + h0 < need && need <= above + h0 + h1) {
        s_bin = b1;
        s_bin_need = need - above - h0;
        s_bin_cnt = h1;
      }
      __syncthreads();
      prefix = (prefix & ~(uint32_t)(((1ull << (hi + 1)) - 1))) |
               ((uint32_t)s_bin << lo);
      need = s_bin_need;
      cnt = s_bin_cnt;
      lo_fixed = lo;
      // The next writes of s_bin* and hist come after further barriers.
    }
    bin_lo = ((uint64_t)prefix >> lo_fixed) << lo_fixed;
    win_lo = bin_lo + (1ull << lo_fixed);
  }
  const uint32_t nwin = (uint32_t)keff - need;
  const bool small_bin = need > 0 && cnt <= (uint32_t)kSmall;
  const bool ordered = need > 0 && !small_bin;   // a run of equal keys

  // Winner buckets of equal width over [max(win_lo, mn), mx], larger keys
  // first.
  const uint32_t wlo = win_lo > (uint64_t)mn ? (uint32_t)min(win_lo, (uint64_t)mx) : mn;
  const uint32_t range = mx - wlo;
  const int shift = range < (uint32_t)kBins ? 0 : (32 - __clz(range)) - 11;
#define bucket_of(KEY) ((int)((mx - (KEY)) >> shift))

  // 3. Histogram of the winners; candidates appended (at most kSmall).
  for (int i = tid; i < kBins; i += NT) hist[i] = 0;
  if (tid == 0) s_nc = 0;
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int base = c * CHUNK;
    if (!RES) ESS_TOPK_LOAD(base);
#pragma unroll
    for (int v = 0; v < VPT; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = pos_of(base, v, e);
        const uint32_t key = kr[4 * v + e];
        if (p < n) {
          if ((uint64_t)key >= win_lo) {
            atomicAdd(&hist[bucket_of(key)], 1u);
          } else if (small_bin && (uint64_t)key >= bin_lo) {
            const uint32_t at = atomicAdd(&s_nc, 1u);
            if (at < (uint32_t)kSmall) cand[at] = full_key(key, p);
          }
        }
      }
  }
  __syncthreads();
  // Bucket starts: thread t owns buckets 2t and 2t+1.
  bool too_big;
  {
    const uint32_t c0 = hist[2 * tid], c1 = hist[2 * tid + 1];
    uint32_t tot;
    const uint32_t off = block_exscan<NT>(c0 + c1, tmp, &tot);
    too_big = __syncthreads_or(max(c0, c1) > (uint32_t)kMaxBucket);
    hist[2 * tid] = off;
    hist[2 * tid + 1] = off + c0;
  }
  __syncthreads();
  // Scatter the winners into their buckets; a run of equal keys in the bin
  // is taken in position order: the positions of slice v are contiguous per
  // thread and ordered by thread, so a workgroup scan gives each its rank.
  uint32_t eq_taken = 0;
  for (int c = 0; c < nchunks; ++c) {
    const int base = c * CHUNK;
    if (!RES) ESS_TOPK_LOAD(base);
#pragma unroll
    for (int v = 0; v < VPT; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = pos_of(base, v, e);
        const uint32_t key = kr[4 * v + e];
        if (p < n && (uint64_t)key >= win_lo) {
          // The histogram bounds every bucket's fill inside [0, nwin).
          const uint32_t at = atomicAdd(&hist[bucket_of(key)], 1u);
          if (at < (uint32_t)kpow2) grp[at] = full_key(key, p);
        }
      }
    if (ordered) {
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        int n_eq = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (pos_of(base, v, e) < n && (uint64_t)kr[4 * v + e] == bin_lo) ++n_eq;
        if (eq_taken < need && __syncthreads_count(n_eq) > 0) {
          uint32_t t2;
          uint32_t rank = eq_taken + block_exscan<NT>(n_eq, tmp, &t2);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int p = pos_of(base, v, e);
            if (p < n && (uint64_t)kr[4 * v + e] == bin_lo) {
              if (rank < need) EMIT(nwin + rank, p, cs[p]);
              ++rank;
            }
          }
          eq_taken += t2;
        }
      }
    }
  }
  __syncthreads();

  // Candidates: the last wave sorts them and writes the best `need`.
  if (small_bin && tid >= NT - 64) {
    const int i = tid - (NT - 64);
    const uint32_t nc = min(s_nc, (uint32_t)kSmall);
    // Real keys carry ~pos >= 2^31 in the low word, so 0 sorts after them.
    const uint64_t x = wave_bitonic_u64<true>(i < (int)nc ? cand[i] : 0ull, i);
    if ((uint32_t)i < need) {
      const int pos = (int)(~(uint32_t)x);
      EMIT(nwin + i, pos, cs[pos]);
    }
  }

  // 4. Winners' ranks.  hist[b] is now the end of bucket b, so bucket b
  // spans [hist[b-1], hist[b]).
  if (!too_big) {
    for (int i = tid; i < (int)nwin; i += NT) {
      const uint64_t x = grp[i];
      const int pos = (int)(~(uint32_t)x);
      const int32_t sl = cs[pos];
      const int bk = bucket_of((uint32_t)(x >> 32));
      const int lo = bk == 0 ? 0 : (int)hist[bk - 1];
      const int hi = (int)hist[bk];
      int r = lo;
      for (int q = lo; q < hi; ++q) r += grp[q] > x;
      EMIT(r, pos, sl);
    }
  } else {
    for (int i = nwin + tid; i < kpow2; i += NT) grp[i] = 0ull;
    __syncthreads();
    block_sort_u64_n<NT, true>(grp, kpow2);
    for (int i = tid; i < (int)nwin; i += NT) {
      const int pos = (int)(~(uint32_t)grp[i]);
      EMIT(i, pos, cs[pos]);
    }
  }
#undef EMIT
#undef bucket_of
#undef pos_of
#undef ESS_TOPK_LOAD
  return keff;
}

template <bool RES>
__global__ __launch_bounds__(NT) void topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ n_vis,
    const int32_t* __restrict__ cache_slots, int32_t* __restrict__ sel_pos,
    int32_t* __restrict__ sel_slot, int32_t* __restrict__ n_sel, int L, int m,
    int n_tok, int k, int kpow2) {
  extern __shared__ uint64_t grp[];  // kpow2: winners grouped by bucket
  topk_row<RES, false>(scores, n_vis, cache_slots, sel_pos, sel_slot, n_sel, L, m,
                       n_tok, k, kpow2, blockIdx.x, grp, nullptr, nullptr);
}

// One query token per request: the top-k and the residency update of a
// request in one workgroup.  The update starts from the selections and
// slots the top-k leaves in LDS, so neither is read back from memory, and
// the step saves a kernel boundary.
template <bool RES>
__global__ __launch_bounds__(NT) void select_update_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ n_vis,
    const int32_t* __restrict__ cache_slots, int32_t* __restrict__ sel_pos,
    int32_t* __restrict__ sel_slot, int32_t* __restrict__ n_sel, int L, int m,
    int k, int kpow2, pool::Args pa, int rank_off) {
  extern __shared__ uint64_t dyn[];  // top-k winners, then the update's entries
  int32_t* rpos = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(dyn) + rank_off);
  int32_t* rslot = rpos + k;
  const int keff = topk_row<RES, true>(scores, n_vis, cache_slots, sel_pos, sel_slot,
                                       n_sel, L, m, 1, k, kpow2, blockIdx.x, dyn,
                                       rpos, rslot);
  __syncthreads();   // ranked selections complete; the winners' buffer is free
  pool::update_request<true>(pa, blockIdx.x, dyn, rpos, rslot, keff);
}

}  // namespace

hipError_t launch_topk(const ess_dims& d, int k, int n_tok,
                       const float* scores, const int32_t* n_vis,
                       const int32_t* cache_slots, int32_t* sel_pos,
                       int32_t* sel_slot, int32_t* n_sel, hipStream_t s) {
  // The fallback sort needs a power of two of at least one key per thread.
  const int kpow2 = pow2_at_least(k) < NT ? NT : pow2_at_least(k);
  const size_t lds = (size_t)kpow2 * sizeof(uint64_t);
  // Rows of at most one chunk stay in registers for all passes.
  const bool res = d.ctx_len <= CHUNK;
  const void* fn = res ? (const void*)topk_kernel<true> : (const void*)topk_kernel<false>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  if (res)
    hipLaunchKernelGGL(topk_kernel<true>, dim3(d.batch * n_tok), dim3(NT), lds, s,
                       scores, n_vis, cache_slots, sel_pos, sel_slot, n_sel,
                       d.ctx_len, d.mtp, n_tok, k, kpow2);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3(d.batch * n_tok), dim3(NT), lds, s,
                       scores, n_vis, cache_slots, sel_pos, sel_slot, n_sel,
                       d.ctx_len, d.mtp, n_tok, k, kpow2);
  return hipGetLastError();
}

bool select_update_fits(const ess_dims& d, int k, int n_tok) {
  return n_tok == 1 && k <= kFusedMaxK;
}

hipError_t launch_select_update(const ess_dims& d, int k, const float* scores,
                                const int32_t* n_vis, int32_t* cache_slots,
                                int32_t* sel_pos, int32_t* sel_slot,
                                int32_t* n_sel, int32_t* slot_pos, void* lru,
                                int32_t* miss_pos, int32_t* miss_slot,
                                int32_t* n_miss, int32_t* n_evict,
                                int32_t* row_dst, int32_t* sel_slot_post,
                                hipStream_t s) {
  const int kpow2 = pow2_at_least(k) < NT ? NT : pow2_at_least(k);
  const int epow2 = kpow2;
  const int two = epow2 <= pool::kTwoBufferMax ? 1 : 0;
  int bits = 0;
  while ((1 << bits) < d.ctx_len) ++bits;
  const int pos_shift = bits > 11 ? bits - 11 : 0;
  const pool::Args pa{sel_pos, n_sel, cache_slots, slot_pos, lru,
                      lru_bytes_per_req(d.pool_slots), miss_pos, miss_slot,
                      n_miss, n_evict, row_dst, sel_slot_post, d.ctx_len,
                      d.pool_slots, k, 1, epow2, two, pos_shift};
  const size_t topk_bytes = (size_t)kpow2 * sizeof(uint64_t);
  const size_t upd_bytes = (size_t)epow2 * sizeof(uint64_t) * (two ? 2 : 1);
  const size_t rank_off = align_up(topk_bytes > upd_bytes ? topk_bytes : upd_bytes, 16);
  const size_t lds = rank_off + 2 * (size_t)k * sizeof(int32_t);
  const bool res = d.ctx_len <= CHUNK;
  const void* fn = res ? (const void*)select_update_kernel<true>
                       : (const void*)select_update_kernel<false>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  if (res)
    hipLaunchKernelGGL(select_update_kernel<true>, dim3(d.batch), dim3(NT), lds, s,
                       scores, n_vis, cache_slots, sel_pos, sel_slot, n_sel,
                       d.ctx_len, d.mtp, k, kpow2, pa, (int)rank_off);
  else
    hipLaunchKernelGGL(select_update_kernel<false>, dim3(d.batch), dim3(NT), lds, s,
                       scores, n_vis, cache_slots, sel_pos, sel_slot, n_sel,
                       d.ctx_len, d.mtp, k, kpow2, pa, (int)rank_off);
  return hipGetLastError();
}

}  // namespace ess
