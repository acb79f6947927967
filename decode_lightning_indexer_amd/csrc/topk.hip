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
//      that bin holds at most `cap` keys (usually after one pass);
//   3. one collect pass: keys above the bin are winners, keys in the bin are
//      candidates; the candidates are sorted in LDS on the full 64-bit key
//      and the best `need` of them join the winners.  If the bin is still
//      too large after all 32 bits (a run of equal scores), the equal keys
//      are taken in position order with a workgroup scan;
//   4. bitonic sort of the k winners (rank order) and the emit pass.
#include "block_util.h"
#include "ess_internal.h"

namespace ess {
namespace {

constexpr int NT = 1024;
constexpr int kBins = 2048;
constexpr size_t kLdsBudget = 160 * 1024 - 16 * 1024;  // leave static LDS room

__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;          // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t full_key(uint32_t ok, int pos) {
  return ((uint64_t)ok << 32) | (uint32_t)(~(uint32_t)pos);
}

__device__ __forceinline__ bool above_fixed(uint32_t key, uint32_t prefix,
                                            int lo_fixed) {
  return ((uint64_t)key >> lo_fixed) > ((uint64_t)prefix >> lo_fixed);
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

template <bool RES>
__global__ __launch_bounds__(NT) void topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ n_vis,
    const int32_t* __restrict__ cache_slots, int32_t* __restrict__ sel_pos,
    int32_t* __restrict__ sel_slot, int32_t* __restrict__ n_sel, int L, int m,
    int n_tok, int k, int kpow2, int cap) {
  extern __shared__ uint64_t smem[];
  uint64_t* win = smem;              // kpow2 winners
  uint64_t* cand = smem + kpow2;     // cap candidates
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t tmp[2 * (NT / 64) + 1];
  __shared__ uint32_t s_bin_need, s_bin_cnt;
  __shared__ int s_bin;

  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int b = row / n_tok, j = row % n_tok;
  const float* srow = scores + ((size_t)b * m + j) * L;
  int n = n_vis[b * m + j];
  n = n < 0 ? 0 : (n > L ? L : n);
  const int keff = min(k, n);
  const bool vec = (L & 3) == 0;     // rows start 16-byte aligned

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

  if (keff == n) {
    // Every visible position is selected.
    for (int i = tid; i < kpow2; i += NT)
      win[i] = i < n ? full_key(ord_key(srow[i]), i) : 0ull;
    __syncthreads();
  } else {
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
    // Bits at and above lo_fixed are common to every key in the bin that
    // holds the k-th key; `prefix` carries them.
    int lo_fixed = (mn == mx) ? 0 : 32 - __clz(mn ^ mx);
    uint32_t prefix = mn;
    uint32_t need = keff;      // keys still to take from the current bin
    uint32_t cnt = n;          // keys in the current bin

    // 2. Radix passes until the bin is small or the bits run out.
    while (cnt > (uint32_t)cap && lo_fixed > 0) {
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
      __syncthreads();
    }

    // 3. Collect winners above the bin and the bin's candidates, compacted
    // with workgroup scans (winner and candidate counts packed in one word:
    // winners <= kpow2 <= 16384 and candidates <= cap fit 16 bits each).
    const bool sort_cands = cnt <= (uint32_t)cap;
    uint32_t eq_taken = 0;  // ordered path: equal keys taken so far
    uint32_t nwin = 0, ncand = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int base = c * CHUNK;
      if (!RES) ESS_TOPK_LOAD(base);
      uint32_t mine = 0;
#pragma unroll
      for (int v = 0; v < VPT; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = kr[4 * v + e];
          if (pos_of(base, v, e) < n) {
            if (above_fixed(key, prefix, lo_fixed)) mine += 1u << 16;
            else if (sort_cands && in_fixed(key, prefix, lo_fixed)) mine += 1u;
          }
        }
      uint32_t tot;
      const uint32_t ex = block_exscan<NT>(mine, tmp, &tot);
      uint32_t wat = nwin + (ex >> 16), cat = ncand + (ex & 0xFFFFu);
#pragma unroll
      for (int v = 0; v < VPT; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = pos_of(base, v, e);
          const uint32_t key = kr[4 * v + e];
          if (p < n) {
            // The counts guarantee wat < kpow2 and cat < cap; the checks
            // only keep LDS writes in bounds if that ever failed.
            if (above_fixed(key, prefix, lo_fixed)) {
              if (wat < (uint32_t)kpow2) win[wat] = full_key(key, p);
              ++wat;
            } else if (sort_cands && in_fixed(key, prefix, lo_fixed)) {
              if (cat < (uint32_t)cap) cand[cat] = full_key(key, p);
              ++cat;
            }
          }
        }
      nwin += tot >> 16;
      ncand += tot & 0xFFFFu;
      if (!sort_cands) {
        // All keys in the bin are equal: take them in position order.  The
        // positions of slice v are contiguous per thread and ordered by
        // thread, so a workgroup scan gives each its rank.
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
          int n_eq = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (pos_of(base, v, e) < n && in_fixed(kr[4 * v + e], prefix, lo_fixed)) ++n_eq;
          if (__syncthreads_count(n_eq) > 0) {
            uint32_t t2;
            uint32_t rank = eq_taken + block_exscan<NT>(n_eq, tmp, &t2);
            uint32_t taken_before = min(eq_taken, need);
            uint32_t at = nwin + (min(rank, need) - taken_before);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int p = pos_of(base, v, e);
              if (p < n && in_fixed(kr[4 * v + e], prefix, lo_fixed)) {
                if (rank < need) {
                  if (at < (uint32_t)kpow2) win[at] = full_key(kr[4 * v + e], p);
                  ++at;
                }
                ++rank;
              }
            }
            const uint32_t before = min(eq_taken, need);
            eq_taken += t2;
            nwin += min(eq_taken, need) - before;
          }
        }
      }
    }
    __syncthreads();
    if (sort_cands) {
      const uint32_t nc = min(ncand, (uint32_t)cap);
      if (nc <= 64) {
        wave_sort_u64<true>(cand, nc, 0ull);
      } else {
        const int cp = max(pow2_at_least_dev(nc), NT);
        for (int i = nc + tid; i < cp; i += NT) cand[i] = 0ull;
        __syncthreads();
        block_sort_u64_n<NT, true>(cand, cp);
      }
      for (uint32_t i = tid; i < need && i < nc && nwin + i < (uint32_t)kpow2; i += NT)
        win[nwin + i] = cand[i];
      __syncthreads();
    }
    for (int i = keff + tid; i < kpow2; i += NT) win[i] = 0ull;
    __syncthreads();
  }

  // 4. Rank order: bucket sort on the score bits spread over the winners'
  // range (buckets of equal-score runs are then ordered by position), or a
  // full sort when the buckets come out uneven or do not fit.
  const uint64_t* ranked = win;
  {
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
    for (int i = tid; i < keff; i += NT) {
      const uint32_t hi = (uint32_t)(win[i] >> 32);
      kmn = min(kmn, hi);
      kmx = max(kmx, hi);
    }
    block_minmax<NT>(kmn, kmx, tmp);
    bool done = false;
    if (cap >= keff) {
      const uint32_t range = kmx - kmn;
      const int shift = range < (uint32_t)kBins ? 0 : (32 - __clz(range)) - 11;
      auto bucket = [&](uint64_t x) {
        return (int)((kmx - (uint32_t)(x >> 32)) >> shift);
      };
      done = bucket_sort_u64<NT, true>(win, cand, keff, kBins, bucket, hist, tmp, 64);
      if (done) ranked = cand;
    }
    if (!done) block_sort_u64_n<NT, true>(win, kpow2);
  }
  int32_t* op = sel_pos + ((size_t)b * n_tok + j) * k;
  int32_t* os = sel_slot + ((size_t)b * n_tok + j) * k;
  const int32_t* cs = cache_slots + (size_t)b * L;
  for (int i = tid; i < k; i += NT) {
    if (i < keff) {
      const int pos = (int)(~(uint32_t)ranked[i]);
      op[i] = pos;
      os[i] = cs[pos];
    } else {
      op[i] = -1;
      os[i] = -1;
    }
  }
  if (tid == 0) n_sel[b * n_tok + j] = keff;
#undef pos_of
#undef ESS_TOPK_LOAD
}

}  // namespace

hipError_t launch_topk(const ess_dims& d, int k, int n_tok,
                       const float* scores, const int32_t* n_vis,
                       const int32_t* cache_slots, int32_t* sel_pos,
                       int32_t* sel_slot, int32_t* n_sel, hipStream_t s) {
  // Sort buffers hold at least one key per thread.
  const int kpow2 = pow2_at_least(k) < NT ? NT : pow2_at_least(k);
  size_t cap = (kLdsBudget - (size_t)kpow2 * 8) / 8;
  if (cap > 4096) cap = 4096;
  int capp = 1;
  while ((size_t)capp * 2 <= cap) capp <<= 1;
  const size_t lds = ((size_t)kpow2 + capp) * sizeof(uint64_t);
  // Rows of at most one chunk stay in registers for all passes.
  const bool res = d.ctx_len <= CHUNK;
  const void* fn = res ? (const void*)topk_kernel<true> : (const void*)topk_kernel<false>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)kLdsBudget);
  if (e != hipSuccess) return e;
  if (res)
    hipLaunchKernelGGL(topk_kernel<true>, dim3(d.batch * n_tok), dim3(NT), lds, s,
                       scores, n_vis, cache_slots, sel_pos, sel_slot, n_sel,
                       d.ctx_len, d.mtp, n_tok, k, kpow2, capp);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3(d.batch * n_tok), dim3(NT), lds, s,
                       scores, n_vis, cache_slots, sel_pos, sel_slot, n_sel,
                       d.ctx_len, d.mtp, n_tok, k, kpow2, capp);
  return hipGetLastError();
}

}  // namespace ess
