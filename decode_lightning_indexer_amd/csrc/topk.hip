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
// A row held in registers (at most 32768 keys) takes steps 3-4 on a compact
// list instead: the selected keys (above the bin, the bin's best `need`, or
// the first `need` of a run of equal keys) are written in position order
// into LDS by packed workgroup scans of per-thread counts, so the k winners
// sit densely in k words; the buckets then rank that list, not the whole
// row.  The list in position order is also what the residency update and
// the tokens of a multi-token step consume (each token's winners by
// position, so the update merges two ordered lists instead of sorting).
//
// Rows longer than one register-resident chunk (32768 keys) and k <= 4096:
// one workgroup per row would stream the row once per pass from one CU
// (~480 us at 1M keys).  Such rows are split over several workgroups that
// run the selection together (see "Rows split over several workgroups"
// below); when the launch would need more workgroups than that allows, the
// row is reduced in levels first.  A level
// splits its input into chunks of 16384, one workgroup each, and writes each
// chunk's exact top-k as (key, position) pairs in ascending position order,
// densely (chunk s at s * k).  The row's top-k lies inside the union of its chunks'
// top-k, so a level loses no winner; levels repeat until at most one chunk
// of candidates is left, and the final workgroup selects from that list as
// above, with positions read from the list.  The candidates stay in
// position order, so "equal keys: lower position first" is still the order
// of the list.
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
constexpr int kLevelMaxK = 4096;  // multi-level selection up to this k (>= 8x per level)
// Rank order by sorting the winners (two kpow2-word LDS buffers) up to this
// power of two; above, the winner buckets rank them (one buffer).
constexpr int kSortRankMax = 4096;

__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;          // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Comparisons as 0/1 register values from min / max / subtract, for tests
// made on every held key.  The keys go through pin() first: an empty asm
// that the compiler cannot look through, so the tests of one key are made
// where they are used, not all at once (with 32 keys per thread the
// compiler otherwise computes every key's lane masks and write values up
// front and spills them).
__device__ __forceinline__ uint32_t pin(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ uint32_t gt_u32(uint32_t a, uint32_t b) {
  return min(max(a, b) - b, 1u);             // 1 iff a > b
}
__device__ __forceinline__ uint32_t ge_u32(uint32_t a, uint32_t b) {
  return 1u - min(max(a, b) - a, 1u);        // 1 iff a >= b
}
__device__ __forceinline__ uint32_t eq_u32(uint32_t a, uint32_t b) {
  return 1u - min(a ^ b, 1u);
}

__device__ __forceinline__ uint64_t full_key(uint32_t ok, int pos) {
  return ((uint64_t)ok << 32) | (uint32_t)(~(uint32_t)pos);
}

// Keys are read in chunks of NT * 32: thread t holds positions
// base + (v * NT + t) * 4 + e for v < 8, e < 4, loaded as eight 16-byte
// loads issued together.  A row of at most one chunk is loaded once and kept
// in registers for every pass (RES); longer rows are streamed per pass.
constexpr int VPT = 8;                 // 16-byte loads per thread per chunk
constexpr int KPT = VPT * 4;           // keys per thread per chunk
constexpr int CHUNK = NT * KPT;        // 32768 keys
// Candidate lists carry a position with each key; both stay in registers
// with half the keys per thread.
constexpr int VPT_E = 4;
constexpr int CHUNK_E = NT * VPT_E * 4;   // 16384 candidates

// One selection input: a run of a scores row (entry i is position pos0 + i)
// or, with EXPL, a candidate list of order-preserving keys with explicit
// positions in ascending order.  n entries; vec: 16-byte aligned start.
// Optionally (a scores row held in registers) the entry count is read from
// n_src instead, clamped to [0, cap], where cap entries of the row are
// allocated: the row is then loaded before its count arrives.
struct RowIn {
  const float* score;
  const uint32_t* key;
  const int32_t* pos;
  int n;
  bool vec;
  int pos0;
  int cap = 0;
  const int32_t* n_src = nullptr;
};

// Rank-order outputs (with the slot of each winner) or, with POSORD, the
// selected (key, position) pairs in input order.
struct RowOut {
  int32_t* op;
  int32_t* os;
  const int32_t* cs;
  int32_t* n_sel;      // may be null
  uint32_t* okey;      // POSORD
  int32_t* opos;       // POSORD
  int32_t* rpos;       // FUSE
  int32_t* rslot;      // FUSE
  // Rank order from a compact list (BYSORT, rows in registers): kpow2 + NT
  // words of LDS that receive the winners' full keys in input order (and
  // one dump word per thread); `grp` then holds them grouped by rank
  // bucket.  With FUSE, rpos / rslot are indexed by that input (= position)
  // order: each winner's rank and slot.
  uint64_t* pw;
  // Optional (BYSORT, not FUSE): the winners in position order for a later
  // residency update - position, rank and slot of each ([k] each).
  int32_t* lpos;
  int32_t* lrank;
  int32_t* lslot;
};

// Rank order of a compact winner list out.pw[0..keff) (full keys in
// ascending position order): buckets of equal key width over [klo, mx],
// larger keys first; a counting pass, a scan, a scatter grouped by bucket,
// then each winner's rank is its bucket's start plus the number of larger
// full keys in its bucket (full keys are unique).  A bucket over kMaxBucket
// keys (long runs of near-equal scores) sorts the whole list instead.  Each
// rank's slot is read from cache_slots; with FUSE each winner's rank and
// slot are also left at its input-order index, and with position lists
// (out.lpos) its position, rank and slot are written there (staged in
// out.rpos / out.rslot with STAGE, then written in order).  grp: kpow2
// words of LDS; the input-order index of each scattered winner goes after
// out.pw's kpow2 + NT words.  hist: kBins words; tmp: scan scratch.
template <bool FUSE, bool STAGE = false>
__device__ __forceinline__ void rank_compact(const RowOut& out, int keff, int kpow2,
                                             uint32_t mx, uint32_t klo, uint64_t* grp,
                                             uint32_t* hist, uint32_t* tmp) {
  const uint64_t* pw = out.pw;
  const int32_t* cs = out.cs;
  int32_t* op = out.op;
  int32_t* os = out.os;
  const int tid = threadIdx.x;
  const uint32_t krange = mx - klo;
  const int kshift = krange < (uint32_t)kBins ? 0 : (32 - __clz(krange)) - 11;
#define rank_bucket(FK) min((int)((mx - (uint32_t)((FK) >> 32)) >> kshift), kBins - 1)
  for (int i = tid; i < kBins; i += NT) hist[i] = 0;
  __syncthreads();
  for (int i = tid; i < keff; i += NT) atomicAdd(&hist[rank_bucket(pw[i])], 1u);
  __syncthreads();
  bool big;
  {
    const uint32_t c0 = hist[2 * tid], c1 = hist[2 * tid + 1];
    uint32_t total;
    const uint32_t off = block_exscan<NT>(c0 + c1, tmp, &total);
    big = __syncthreads_or(max(c0, c1) > (uint32_t)kMaxBucket);
    hist[2 * tid] = off;
    hist[2 * tid + 1] = off + c0;
  }
  __syncthreads();
  // pidx[j]: the input-order index of grp[j] (FUSE or position lists), so
  // each rank finds its winner's place in the position-ordered list
  // directly.
  const bool lists = FUSE || out.lpos != nullptr;
  constexpr bool stage = !FUSE && STAGE;
  uint32_t* pidx = reinterpret_cast<uint32_t*>(out.pw + kpow2 + NT);
  auto emit_rank = [&](int r, uint64_t x, int i) {
    const int pos = (int)(~(uint32_t)x);     // -1 only for "no winner"
    const int32_t sl = pos >= 0 ? cs[pos] : -1;
    op[r] = pos;
    os[r] = sl;
    if (lists) {
      if (i < 0) {                           // (the full sort: search)
        int lo = 0, hi = keff - 1;           // pw ascends in position
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if ((int)(~(uint32_t)pw[mid]) < pos) lo = mid + 1;
          else hi = mid;
        }
        i = lo;
      }
      if (FUSE || stage) {
        out.rpos[i] = r;
        out.rslot[i] = sl;
      } else {
        out.lpos[i] = pos;
        out.lrank[i] = r;
        out.lslot[i] = sl;
      }
    }
  };
  if (!big) {
    for (int i = tid; i < keff; i += NT) {
      const uint64_t x = pw[i];
      const uint32_t at = atomicAdd(&hist[rank_bucket(x)], 1u);
      grp[at] = x;
      if (lists) pidx[at] = (uint32_t)i;
    }
    __syncthreads();
    // hist[b] is now the end of bucket b: bucket b spans [hist[b-1], hist[b]).
    for (int j = tid; j < keff; j += NT) {
      const uint64_t x = grp[j];
      const int bk = rank_bucket(x);
      const int lo = bk == 0 ? 0 : (int)hist[bk - 1];
      const int hi = (int)hist[bk];
      int r = lo;
      for (int q = lo; q < hi; ++q) r += grp[q] > x;
      emit_rank(r, x, lists ? (int)pidx[j] : -1);
    }
  } else {
    for (int i = tid; i < kpow2; i += NT) grp[i] = i < keff ? pw[i] : 0ull;
    __syncthreads();
    block_sort_u64_n<NT, true>(grp, kpow2);
    for (int r = tid; r < keff; r += NT) emit_rank(r, grp[r], -1);
  }
  if (stage && lists) {
    __syncthreads();
    for (int i = tid; i < keff; i += NT) {
      out.lpos[i] = (int)(~(uint32_t)pw[i]);
      out.lrank[i] = out.rpos[i];
      out.lslot[i] = out.rslot[i];
    }
  }
#undef rank_bucket
}

// Top-k of one input by a 1024-thread workgroup; returns the number
// selected.  grp: kpow2 winners of LDS (rank order only).  FUSE: the
// outputs are also left in LDS (rpos, rslot) for the residency update that
// follows in the same workgroup.
template <bool RES, bool FUSE, bool EXPL, bool POSORD, int TVX = 0, bool BYSORT = false>
__device__ __forceinline__ int topk_row(const RowIn& in, int k, int kpow2, const RowOut& out,
                        uint64_t* grp) {
  static_assert(!POSORD || RES, "position-order output needs the row in registers");
  static_assert(!BYSORT || (RES && !POSORD), "rank order by sort needs the row in registers");
  __shared__ uint32_t hist[kBins];
  __shared__ uint64_t cand[kSmall];
  __shared__ uint32_t tmp[2 * (NT / 64) + 1];
  __shared__ uint32_t s_bin_need, s_bin_cnt, s_nc;
  __shared__ int s_bin;
  __shared__ uint64_t s_thr;
  __shared__ uint64_t tmp64[NT / 64 + 1];
  // Keys per thread: candidate lists hold half as many, with positions.
  constexpr int TV = TVX ? TVX : (EXPL ? VPT_E : VPT);
  constexpr int TK = TV * 4;
  constexpr int TC = NT * TK;

  const int tid = threadIdx.x;
  const float* srow = in.score;
  const uint32_t* krow = in.key;
  const int32_t* prow = in.pos;
  const int pos0 = in.pos0;
  const bool vec = in.vec;
  // Keys of one chunk for this thread, of the first LIM entries.  A chunk
  // wholly inside them (the common case) takes eight unconditional 16-byte
  // loads, all in flight together; a partial chunk takes bounds-checked
  // scalar loads (zero past LIM).
  uint32_t kr[TK];
  int32_t pr[TK];   // positions of a candidate list's keys (EXPL only)
#define ESS_TOPK_LOAD(BASE, LIM)                                                   \
  do {                                                                        \
    const int base_ = (BASE);                                                 \
    if (vec && base_ + TC <= (LIM)) {                                          \
      if constexpr (EXPL) {                                                   \
        uint4 a_[TV];                                                         \
        int4 q_[TV];                                                          \
        _Pragma("unroll") for (int v = 0; v < TV; ++v) {                      \
          a_[v] = *reinterpret_cast<const uint4*>(krow + base_ + (v * NT + tid) * 4); \
          q_[v] = *reinterpret_cast<const int4*>(prow + base_ + (v * NT + tid) * 4);  \
        }                                                                     \
        _Pragma("unroll") for (int v = 0; v < TV; ++v) {                      \
          kr[4 * v + 0] = a_[v].x;                                            \
          kr[4 * v + 1] = a_[v].y;                                            \
          kr[4 * v + 2] = a_[v].z;                                            \
          kr[4 * v + 3] = a_[v].w;                                            \
          pr[4 * v + 0] = q_[v].x;                                            \
          pr[4 * v + 1] = q_[v].y;                                            \
          pr[4 * v + 2] = q_[v].z;                                            \
          pr[4 * v + 3] = q_[v].w;                                            \
        }                                                                     \
      } else {                                                                \
        float4 f_[TV];                                                       \
        _Pragma("unroll") for (int v = 0; v < TV; ++v)                       \
          f_[v] = *reinterpret_cast<const float4*>(srow + base_ + (v * NT + tid) * 4); \
        _Pragma("unroll") for (int v = 0; v < TV; ++v) {                     \
          kr[4 * v + 0] = ord_key(f_[v].x);                                   \
          kr[4 * v + 1] = ord_key(f_[v].y);                                   \
          kr[4 * v + 2] = ord_key(f_[v].z);                                   \
          kr[4 * v + 3] = ord_key(f_[v].w);                                   \
        }                                                                     \
      }                                                                       \
    } else {                                                                  \
      _Pragma("unroll") for (int v = 0; v < TV; ++v)                         \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) {                       \
          const int p_ = base_ + (v * NT + tid) * 4 + e;                      \
          if constexpr (EXPL) {                                               \
            kr[4 * v + e] = p_ < (LIM) ? krow[p_] : 0u;                       \
            pr[4 * v + e] = p_ < (LIM) ? prow[p_] : 0;                        \
          } else {                                                            \
            kr[4 * v + e] = p_ < (LIM) ? ord_key(srow[p_]) : 0u;              \
          }                                                                   \
        }                                                                     \
    }                                                                         \
  } while (0)
  // A scores row held in registers whose entry count comes from memory:
  // the count's load goes first, then the row's (bounded by the allocated
  // cap), and only then is the count waited for, so the two round trips
  // overlap; keys past the count are zeroed as the bounded loads leave them.
  const bool early = RES && !EXPL && in.n_src != nullptr;
  int n_in = in.n;
  if (early) {
    n_in = *in.n_src;
    ESS_TOPK_LOAD(0, in.cap);
  }
  const int n = early ? min(max(n_in, 0), in.cap) : n_in;
  if (early) {
#pragma unroll
    for (int v = 0; v < TV; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((v * NT + tid) * 4 + e >= n) kr[4 * v + e] = 0u;
  }
  const int keff = min(k, n);
  int32_t* op = out.op;
  int32_t* os = out.os;
  const int32_t* cs = out.cs;
  if (!POSORD) {
    for (int i = keff + tid; i < k; i += NT) {
      op[i] = -1;
      os[i] = -1;
    }
    if (tid == 0 && out.n_sel) *out.n_sel = keff;
  }
  if (keff == 0) return 0;
  // Output row r: the selection and its slot.
#define EMIT(R, POS, SLOT)                                                    \
  do {                                                                        \
    op[R] = (POS);                                                            \
    os[R] = (SLOT);                                                           \
    if (FUSE) {                                                               \
      out.rpos[R] = (POS);                                                    \
      out.rslot[R] = (SLOT);                                                  \
    }                                                                         \
  } while (0)

  // Index of a held key in the input, and its position.
#define pos_of(BASE, V, E) ((BASE) + ((V) * NT + tid) * 4 + (E))
#define real_pos(BASE, V, E) (EXPL ? pr[4 * (V) + (E)] : pos0 + pos_of(BASE, V, E))
  const int nchunks = (n + TC - 1) / TC;

  if (RES && !early) ESS_TOPK_LOAD(0, n);
  // 1. Range of the keys.
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int c = 0; c < nchunks; ++c) {
    const int base = c * TC;
    if (!RES) ESS_TOPK_LOAD(base, n);
#pragma unroll
    for (int v = 0; v < TV; ++v)
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
      // Keys in the current bin share the bits at and above lo_fixed
      // (32-bit test; lo_fixed = 32 lets every key through).
      const uint32_t fixed_mask = lo_fixed >= 32 ? 0u : (~0u << lo_fixed);
      for (int c = 0; c < nchunks; ++c) {
        const int base = c * TC;
        if (!RES) ESS_TOPK_LOAD(base, n);
#pragma unroll
        for (int v = 0; v < TV; ++v)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t key = pin(kr[4 * v + e]);
            if (pos_of(base, v, e) < n && ((key ^ prefix) & fixed_mask) == 0u)
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

  constexpr bool by_sort = BYSORT;
  if constexpr (by_sort) {
    // Every slot the emission below does not write reads as "no winner".
    for (int i = tid; i < kpow2; i += NT) out.pw[i] = 0ull;
    __syncthreads();
  }
  // 32-bit forms of the bin bounds: keys above the bin are >= win32 (none
  // when win_lo = 2^32), keys in it are >= bin32.
  const bool win_any = win_lo <= 0xFFFFFFFFull;
  const uint32_t win32 = (uint32_t)win_lo, bin32 = (uint32_t)bin_lo;
  if constexpr (POSORD || by_sort) {
    // The selected pairs in input order: keys above the bin; of a small bin
    // the `need` largest full keys (one wave sorts the bin, the need-th
    // becomes a threshold); of a run of equal keys the first `need`.
    if (small_bin) {
      if (tid == 0) s_nc = 0;
      __syncthreads();
      for (int c = 0; c < nchunks; ++c) {
        const int base = c * TC;
        if (!RES) ESS_TOPK_LOAD(base, n);
#pragma unroll
        for (int v = 0; v < TV; ++v)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t key = pin(kr[4 * v + e]);
            if (pos_of(base, v, e) < n && key >= bin32 && (!win_any || key < win32)) {
              const uint32_t at = atomicAdd(&s_nc, 1u);
              if (at < (uint32_t)kSmall) cand[at] = full_key(key, real_pos(base, v, e));
            }
          }
      }
      __syncthreads();
      if (tid >= NT - 64) {
        const int i = tid - (NT - 64);
        const uint32_t nc = min(s_nc, (uint32_t)kSmall);
        const uint64_t x = wave_bitonic_u64<true>(i < (int)nc ? cand[i] : 0ull, i);
        if ((uint32_t)i == need - 1) s_thr = x;
      }
      __syncthreads();
    }
    const uint64_t thr = small_bin ? s_thr : 0ull;
    const uint32_t thr_key = (uint32_t)(thr >> 32), thr_npos = (uint32_t)thr;
    // Index order is group-major (v, then thread, then e): the counts of a
    // thread's groups go through packed scans, 16 bits per group, four
    // groups per 64-bit word.
    constexpr int NW = (TV + 3) / 4;
#define ESS_FIELD(W, V) ((uint32_t)(((W)[(V) >> 2] >> (16 * ((V) & 3))) & 0xFFFFu))
    uint32_t at = 0;   // uniform
    for (int c = 0; c < nchunks; ++c) {
      const int base = c * TC;
      if (!RES) ESS_TOPK_LOAD(base, n);
      // Ranks of equal keys in a run (first `need` in index order win).
      uint32_t eqr[TV];
#pragma unroll
      for (int v = 0; v < TV; ++v) eqr[v] = need;
      if (ordered) {
        uint64_t pk[NW], pre[NW], tot[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) pk[w] = 0;
#pragma unroll
        for (int v = 0; v < TV; ++v) {
          uint64_t n_eq = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            n_eq += (pos_of(base, v, e) < n && kr[4 * v + e] == bin32) ? 1u : 0u;
          pk[v >> 2] |= n_eq << (16 * (v & 3));
        }
#pragma unroll
        for (int w = 0; w < NW; ++w) pre[w] = block_exscan_u64<NT>(pk[w], tmp64, &tot[w]);
        uint32_t acc = 0;
#pragma unroll
        for (int v = 0; v < TV; ++v) {
          eqr[v] = acc + ESS_FIELD(pre, v);
          acc += ESS_FIELD(tot, v);
        }
        // (equal keys of earlier chunks precede; a single chunk here)
      }
      // Selection flags without divergent branches (small_bin and ordered
      // are uniform): of a small bin the full keys from the threshold up
      // (every key above the bin is larger), of a run of equal keys the
      // first `need`, otherwise the keys above the bin.
      uint32_t selm = 0;
      uint64_t sk[NW], pre[NW], tot[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) sk[w] = 0;
      // One loop per case, so no case's tests are evaluated for another's.
      // Keys above the bin: none when win_lo = 2^32 (win32 = 0 then, and
      // win_mul = 0 cancels the test).
      const uint32_t win_mul = win_any ? 1u : 0u;
#define ESS_SEL_LOOP(TEST)                                                     \
  _Pragma("unroll") for (int v = 0; v < TV; ++v) {                             \
    uint32_t cv = 0;                                                           \
    _Pragma("unroll") for (int e = 0; e < 4; ++e) {                            \
      const uint32_t key = pin(kr[4 * v + e]);                                 \
      const uint32_t inr = gt_u32((uint32_t)n, (uint32_t)pos_of(base, v, e));  \
      const uint32_t t = inr & (TEST);                                         \
      selm |= t << (4 * v + e);                                                \
      cv += t;                                                                 \
    }                                                                          \
    sk[v >> 2] |= (uint64_t)cv << (16 * (v & 3));                              \
  }
      if (small_bin) {
        ESS_SEL_LOOP(gt_u32(key, thr_key) |
                     (eq_u32(key, thr_key) & ge_u32(~(uint32_t)real_pos(base, v, e), thr_npos)))
      } else if (ordered) {
#pragma unroll
        for (int v = 0; v < TV; ++v) {
          uint32_t cv = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t key = pin(kr[4 * v + e]);
            const uint32_t inr = gt_u32((uint32_t)n, (uint32_t)pos_of(base, v, e));
            const uint32_t eq = inr & eq_u32(key, bin32);
            const uint32_t t = (inr & win_mul & ge_u32(key, win32)) |
                               (eq & gt_u32(need, eqr[v]));
            eqr[v] += eq;
            selm |= t << (4 * v + e);
            cv += t;
          }
          sk[v >> 2] |= (uint64_t)cv << (16 * (v & 3));
        }
      } else {
        ESS_SEL_LOOP(win_mul & ge_u32(key, win32))
      }
#undef ESS_SEL_LOOP
#pragma unroll
      for (int w = 0; w < NW; ++w) pre[w] = block_exscan_u64<NT>(sk[w], tmp64, &tot[w]);
#pragma unroll
      for (int v = 0; v < TV; ++v) {
        uint32_t o = at + ESS_FIELD(pre, v);
        if constexpr (POSORD) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((selm >> (4 * v + e)) & 1u) {
              if (o < (uint32_t)keff) {   // exactly keff are selected
                out.okey[o] = kr[4 * v + e];
                out.opos[o] = real_pos(base, v, e);
              }
              ++o;
            }
        } else {
          // Every key is written, without a branch: a winner at its place,
          // the others to this thread's own slot past the list.
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t key = pin(kr[4 * v + e]);
            const uint32_t sel = (selm >> (4 * v + e)) & 1u;
            const uint32_t dst = sel && o < (uint32_t)keff ? o : (uint32_t)(kpow2 + tid);
            out.pw[dst] = full_key(key, real_pos(base, v, e));
            o += sel;
          }
        }
        at += ESS_FIELD(tot, v);
      }
    }
#undef ESS_FIELD
    if constexpr (POSORD) return keff;
  }
  if constexpr (by_sort) {
    __syncthreads();
    const uint32_t klo = max(need > 0 ? (uint32_t)bin_lo : (uint32_t)min(win_lo, (uint64_t)mx), mn);
    rank_compact<FUSE>(out, keff, kpow2, mx, klo, grp, hist, tmp);
    return keff;
  } else if constexpr (!POSORD) {

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
    const int base = c * TC;
    if (!RES) ESS_TOPK_LOAD(base, n);
#pragma unroll
    for (int v = 0; v < TV; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = pos_of(base, v, e);
        const uint32_t key = kr[4 * v + e];
        if (p < n) {
          if ((uint64_t)key >= win_lo) {
            atomicAdd(&hist[bucket_of(key)], 1u);
          } else if (small_bin && (uint64_t)key >= bin_lo) {
            const uint32_t at = atomicAdd(&s_nc, 1u);
            if (at < (uint32_t)kSmall) cand[at] = full_key(key, real_pos(base, v, e));
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
    const int base = c * TC;
    if (!RES) ESS_TOPK_LOAD(base, n);
#pragma unroll
    for (int v = 0; v < TV; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = pos_of(base, v, e);
        const uint32_t key = kr[4 * v + e];
        if (p < n && (uint64_t)key >= win_lo) {
          // The histogram bounds every bucket's fill inside [0, nwin).
          const uint32_t at = atomicAdd(&hist[bucket_of(key)], 1u);
          if (at < (uint32_t)kpow2) grp[at] = full_key(key, real_pos(base, v, e));
        }
      }
    if (ordered) {
#pragma unroll
      for (int v = 0; v < TV; ++v) {
        int n_eq = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (pos_of(base, v, e) < n && (uint64_t)kr[4 * v + e] == bin_lo) ++n_eq;
        if (eq_taken < need && __syncthreads_count(n_eq) > 0) {
          uint32_t t2;
          uint32_t rank = eq_taken + block_exscan<NT>(n_eq, tmp, &t2);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (pos_of(base, v, e) < n && (uint64_t)kr[4 * v + e] == bin_lo) {
              const int p = real_pos(base, v, e);
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
#undef real_pos
#undef ESS_TOPK_LOAD
  return keff;
  }
  return keff;   // (position-order output returned above)
}

// Candidates a level leaves of n entries: k per full chunk and min(k, rest)
// of the last (k <= chunk).  Every level reads its input (the scores, then
// candidate lists) in chunks of CHUNK_E, 16 keys per thread: a workgroup's
// passes cost less with fewer keys per thread, and twice the workgroups
// share the row (measured at 128K: 63 -> 37 us against 32768-key chunks).
__host__ __device__ __forceinline__ int level_chunk(int level) {
  (void)level;
  return CHUNK_E;
}
__host__ __device__ __forceinline__ int level_count(int n, int k, int level) {
  const int c = level_chunk(level);
  return (n / c) * k + min(k, n % c);
}

__device__ __forceinline__ int visible(const int32_t* n_vis, int b, int m, int j,
                                       int L) {
  const int n = n_vis[b * m + j];
  return n < 0 ? 0 : (n > L ? L : n);
}

template <bool RES, bool BYSORT>
__global__ __launch_bounds__(NT) void topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ n_vis,
    const int32_t* __restrict__ cache_slots, int32_t* __restrict__ sel_pos,
    int32_t* __restrict__ sel_slot, int32_t* __restrict__ n_sel, int L, int m,
    int n_tok, int k, int kpow2, PosLists pl) {
  // kpow2 words: winners grouped by bucket, or (rank order by sort) the sort
  // buffer followed by kpow2 words for the winners in position order.
  extern __shared__ uint64_t grp[];
  const int row = blockIdx.x, b = row / n_tok, j = row % n_tok;
  const size_t o = ((size_t)b * n_tok + j) * k;
  // (a row held in registers reads its visible count inside, with its loads
  // already issued)
  const RowIn in{scores + ((size_t)b * m + j) * L, nullptr, nullptr,
                 RES ? 0 : visible(n_vis, b, m, j, L), (L & 3) == 0, 0,
                 L, RES ? n_vis + b * m + j : nullptr};
  const RowOut out{sel_pos + o, sel_slot + o, cache_slots + (size_t)b * L,
                   n_sel + b * n_tok + j, nullptr, nullptr, nullptr, nullptr,
                   BYSORT ? grp + kpow2 : nullptr,
                   pl.pos ? pl.pos + o : nullptr, pl.pos ? pl.rank + o : nullptr,
                   pl.pos ? pl.slot + o : nullptr};
  topk_row<RES, false, false, false, 0, BYSORT>(in, k, kpow2, out, grp);
}

// One level of a long row's reduction: workgroup (s, row) writes the exact
// top-k of chunk s of the row's current list as (key, position) pairs in
// position order at s * k of the next list.  Level 1 reads the scores.
template <bool EXPL>
__global__ __launch_bounds__(NT) void topk_level_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ n_vis,
    const uint32_t* __restrict__ ikey, const int32_t* __restrict__ ipos,
    uint32_t* __restrict__ okey, int32_t* __restrict__ opos, size_t cap, int L,
    int m, int n_tok, int k, int kpow2, int level) {
  const int row = blockIdx.y, b = row / n_tok, j = row % n_tok;
  int n = visible(n_vis, b, m, j, L);
  for (int l = 1; l < level; ++l) n = level_count(n, k, l);
  constexpr int kChunk = CHUNK_E;
  const int base = blockIdx.x * kChunk;
  if (base >= n) return;      // this row's list is shorter
  const int ns = min(kChunk, n - base);
  const size_t rb = (size_t)row * cap;
  RowIn in;
  if constexpr (EXPL)
    in = RowIn{nullptr, ikey + rb + base, ipos + rb + base, ns,
               ((rb + base) & 3) == 0, 0};
  else
    in = RowIn{scores + ((size_t)b * m + j) * L + base, nullptr, nullptr, ns,
               (L & 3) == 0, base};
  const size_t ob = rb + (size_t)blockIdx.x * k;
  // (Staging this output in LDS to write it without a branch per key was
  // measured slower: 13.4 -> 14.0 us and 13.9 -> 15.8 us per level at 1M.)
  const RowOut out{nullptr, nullptr, nullptr, nullptr, okey + ob, opos + ob,
                   nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  topk_row<true, false, EXPL, true, VPT_E>(in, k, kpow2, out, nullptr);
}

// The final selection of a long row from its candidate list after `levels`
// levels: rank order with slots.
template <bool BYSORT>
__global__ __launch_bounds__(NT) void topk_final_kernel(
    const uint32_t* __restrict__ ckey, const int32_t* __restrict__ cpos,
    size_t cap, const int32_t* __restrict__ n_vis,
    const int32_t* __restrict__ cache_slots, int32_t* __restrict__ sel_pos,
    int32_t* __restrict__ sel_slot, int32_t* __restrict__ n_sel, int L, int m,
    int n_tok, int k, int kpow2, int levels, PosLists pl) {
  extern __shared__ uint64_t grp[];
  const int row = blockIdx.x, b = row / n_tok, j = row % n_tok;
  int n = visible(n_vis, b, m, j, L);
  for (int l = 1; l <= levels; ++l) n = level_count(n, k, l);
  const size_t rb = (size_t)row * cap, o = ((size_t)b * n_tok + j) * k;
  const RowIn in{nullptr, ckey + rb, cpos + rb, n, (rb & 3) == 0, 0};
  const RowOut out{sel_pos + o, sel_slot + o, cache_slots + (size_t)b * L,
                   n_sel + b * n_tok + j, nullptr, nullptr, nullptr, nullptr,
                   BYSORT ? grp + kpow2 : nullptr,
                   pl.pos ? pl.pos + o : nullptr, pl.pos ? pl.rank + o : nullptr,
                   pl.pos ? pl.slot + o : nullptr};
  topk_row<true, false, true, false, 0, BYSORT>(in, k, kpow2, out, grp);
}

// One query token per request: the top-k and the residency update of a
// request in one workgroup.  The update starts from the selections and
// slots the top-k leaves in LDS, so neither is read back from memory, and
// the step saves a kernel boundary.  With levels > 0 the top-k reads the
// request's candidate list instead of its scores.
template <bool RES, bool EXPL>
__global__ __launch_bounds__(NT) void select_update_kernel(
    const float* __restrict__ scores, const uint32_t* __restrict__ ckey,
    const int32_t* __restrict__ cpos, size_t cap,
    const int32_t* __restrict__ n_vis, const int32_t* __restrict__ cache_slots,
    int32_t* __restrict__ sel_pos, int32_t* __restrict__ sel_slot,
    int32_t* __restrict__ n_sel, int L, int m, int k, int kpow2, int levels,
    pool::Args pa, int rank_off) {
  // Top-k: the sort buffer, then the winners in position order (kpow2 words
  // each); then the update's entries over the sort buffer.  rpos / rslot:
  // per winner its rank and slot (in position order after a sort, in rank
  // order otherwise).
  extern __shared__ uint64_t dyn[];
  int32_t* rpos = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(dyn) + rank_off);
  int32_t* rslot = rpos + k;
  const int b = blockIdx.x;
  const size_t o = (size_t)b * k;
  // Rows held in registers rank their winners by a sort and hand the update
  // a position-ordered selection (it then sorts nothing).
  constexpr bool kSorted = RES;
  uint64_t* pw = kSorted ? dyn + kpow2 : nullptr;
  const RowOut out{sel_pos + o, sel_slot + o, cache_slots + (size_t)b * L, n_sel + b,
                   nullptr, nullptr, rpos, rslot, pw, nullptr, nullptr, nullptr};
  int keff;
  if constexpr (EXPL) {
    int n = visible(n_vis, b, m, 0, L);
    for (int l = 1; l <= levels; ++l) n = level_count(n, k, l);
    const size_t rb = (size_t)b * cap;
    const RowIn in{nullptr, ckey + rb, cpos + rb, n, (rb & 3) == 0, 0};
    keff = topk_row<true, true, true, false, 0, kSorted>(in, k, kpow2, out, dyn);
  } else {
    // (a row held in registers reads its visible count inside, with its
    // loads already issued)
    const RowIn in{scores + (size_t)b * m * L, nullptr, nullptr,
                   RES ? 0 : visible(n_vis, b, m, 0, L), (L & 3) == 0, 0,
                   L, RES ? n_vis + b * m : nullptr};
    keff = topk_row<RES, true, false, false, 0, kSorted>(in, k, kpow2, out, dyn);
  }
  __syncthreads();   // selections complete; the sort buffer is free
  if constexpr (kSorted)
    pool::update_request<true, true>(pa, b, dyn, rpos, rslot, keff, pw);
  else
    pool::update_request<true>(pa, b, dyn, rpos, rslot, keff);
}

// ---------------------------------------------------------------------------
// Rows split over several workgroups.  A row over one register chunk is cut
// into spans of CHUNK_E keys, one workgroup each, held in registers for the
// whole kernel; the workgroups of a row run the radix select together and
// meet at row barriers between its phases:
//   1. a window that holds every winner: each thread's largest key goes
//      into a histogram over the keys' top 11 bits, merged over the row
//      (device atomics); the bin holding the k-th largest of these thread
//      maxima starts the window - they are keys, so at least k keys lie at
//      or above that bin's lower edge, which is therefore no higher than the
//      k-th key - and the highest non-empty bin ends it;
//   2. radix passes of 11 bits over the window, from the first bit where its
//      ends differ (only keys in the window are counted, a small share of
//      the row): each span adds its histogram into the row's, and after the
//      barrier every span picks the same bin holding the k-th key, until
//      that bin holds at most one wave's worth of keys or the bits run out;
//   3. each span publishes how many of its keys lie above and in the final
//      bin (and, for a small bin, the bin's keys themselves); after the
//      barrier every span knows the winners of every span, so its own
//      winners' offset in the row's position-ordered winner list;
//   4. each span writes its winners there, in position order;
//   5. the last span of the row to finish ranks the list (as one workgroup
//      ranks a compact list) and, with one token per request, runs the
//      residency update.
// Data that cross workgroups are written and read with device-scope atomic
// stores and loads, which stay coherent across the XCDs' L2 caches without a
// write-back or invalidation of either cache; each wave waits for its own
// stores before its workgroup arrives at a barrier.  A barrier needs every
// workgroup of the row resident at once: a launch has at most half as many
// workgroups as the device has compute units (so two such launches in flight
// still fit), and every wait is bounded - past kSplitSpin polls the row is
// marked broken, the workgroups run on, and the row is reported with no
// selection (n_sel = 0; with the update fused, the request's LRU error 3).
constexpr int kSplitBits = 11;
constexpr int kSplitBins = 1 << kSplitBits;   // = kBins: the local histogram reuses hist
constexpr int kSplitPasses = (32 + kSplitBits - 1) / kSplitBits;
constexpr int kSplitMaxSpans = 256;
constexpr uint32_t kSplitSpin = 1u << 21;
// Control words of a row, each on its own 128-byte line.
constexpr int kCtlArrive = 0, kCtlDone = 32, kCtlCand = 64, kCtlBroken = 96;
constexpr int kCtlWords = 128;

// Per-row layout of the split selection's workspace (bytes): control words,
// the window's and the passes' histograms (cleared before each launch), then
// per span (keys above the final bin, keys in it), the small final bin's
// keys, and the winners in position order.
struct SplitLayout {
  size_t hist, mm, cand, win, clear_words, row_bytes;
};
inline SplitLayout split_layout(int spans, int k) {
  SplitLayout l;
  l.hist = kCtlWords * 4;
  l.mm = l.hist + (size_t)(1 + kSplitPasses) * kSplitBins * 4;
  l.clear_words = l.mm / 4;   // a multiple of four (the clear kernel's 16-byte stores)
  l.cand = l.mm + align_up((size_t)spans * 8, 128);
  l.win = l.cand + (size_t)kSmall * 8;
  l.row_bytes = align_up(l.win + (size_t)k * 8, 256);
  return l;
}

__device__ __forceinline__ void dev_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void dev_store64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t dev_load(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t dev_load64(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t dev_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// This wave's memory operations complete (stores acknowledged) before any
// later one issues.
__device__ __forceinline__ void wait_own_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Row barrier number `phase` (1, 2, ...): every workgroup of the row
// arrives once per phase.
__device__ __forceinline__ void row_barrier(uint32_t* ctl, uint32_t phase, int spans) {
  wait_own_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    dev_add(ctl + kCtlArrive, 1u);
    const uint32_t target = phase * (uint32_t)spans;
    uint32_t polls = 0;
    while (dev_load(ctl + kCtlArrive) < target) {
      if (++polls > kSplitSpin) {
        dev_add(ctl + kCtlBroken, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// Zero the first `words` 32-bit words of every row (a multiple of four):
// blockIdx.y = row, blockIdx.x = one of gridDim.x slices, 16-byte stores.
__global__ __launch_bounds__(256) void split_clear_kernel(char* sws, size_t row_bytes,
                                                          int words) {
  uint4* p = reinterpret_cast<uint4*>(sws + (size_t)blockIdx.y * row_bytes);
  const int n = words / 4;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct SplitArgs {
  const float* scores;
  const int32_t* n_vis;
  const int32_t* cache_slots;
  int32_t* sel_pos;
  int32_t* sel_slot;
  int32_t* n_sel;
  char* sws;
  size_t row_bytes;
  SplitLayout lay;
  PosLists pl;
  int L, m, n_tok, k, kpow2, rank_off;
};

template <bool FUSE>
__global__ __launch_bounds__(NT) void topk_split_kernel(SplitArgs a, pool::Args pa) {
  extern __shared__ uint64_t dyn[];
  __shared__ uint32_t hist[kBins];             // this span's pass histogram, then ranks
  __shared__ uint32_t tmp[2 * (NT / 64) + 1];
  __shared__ uint64_t tmp64[NT / 64 + 1];
  __shared__ uint32_t s_win[kSplitMaxSpans];   // small bin: winners per span
  __shared__ int s_bin;
  __shared__ uint32_t s_bin_need, s_bin_cnt, s_above, s_off, s_nc, s_prefix, s_need, s_last;
  __shared__ uint64_t s_thr;
  constexpr int TV = VPT_E, TK = TV * 4, S = CHUNK_E;
  static_assert(TV == 4, "the emission packs four 16-bit group counts in 64 bits");
  const int tid = threadIdx.x, g = blockIdx.x, spans = gridDim.x, row = blockIdx.y;
  const int b = row / a.n_tok, j = row % a.n_tok;
  char* rw = a.sws + (size_t)row * a.row_bytes;
  uint32_t* ctl = reinterpret_cast<uint32_t*>(rw);
  uint32_t* rhist = reinterpret_cast<uint32_t*>(rw + a.lay.hist);
  uint32_t* mm = reinterpret_cast<uint32_t*>(rw + a.lay.mm);
  uint64_t* gcand = reinterpret_cast<uint64_t*>(rw + a.lay.cand);
  uint64_t* gwin = reinterpret_cast<uint64_t*>(rw + a.lay.win);
  const int L = a.L, k = a.k;
  const int n = visible(a.n_vis, b, a.m, j, L);
  const int keff = min(k, n);
  const int base = g * S;
  const float* srow = a.scores + ((size_t)b * a.m + j) * L;
#define sp_pos(V, E) (base + ((V) * NT + tid) * 4 + (E))

  // This span's keys, in registers for the whole kernel.
  uint32_t kr[TK];
  if ((L & 3) == 0 && base + S <= n) {
    float4 f[TV];
#pragma unroll
    for (int v = 0; v < TV; ++v)
      f[v] = *reinterpret_cast<const float4*>(srow + sp_pos(v, 0));
#pragma unroll
    for (int v = 0; v < TV; ++v) {
      kr[4 * v + 0] = ord_key(f[v].x);
      kr[4 * v + 1] = ord_key(f[v].y);
      kr[4 * v + 2] = ord_key(f[v].z);
      kr[4 * v + 3] = ord_key(f[v].w);
    }
  } else {
#pragma unroll
    for (int v = 0; v < TV; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = sp_pos(v, e);
        kr[4 * v + e] = p < n ? ord_key(srow[p]) : 0u;
      }
  }

  // 1. The window: a histogram of the thread maxima over the top 11 bits.
  const bool all = keff >= n;
  uint32_t my_above = 0;
  const uint32_t my_vis = n > base ? (uint32_t)min(n - base, S) : 0u;
  uint32_t my_inbin = my_vis;
  uint64_t bin_lo = 0, win_lo = 0;
  uint32_t need = 0, cnt = 0;
  uint32_t phase = 1;
  if (!all) {
    uint32_t tm = 0, has = 0;
#pragma unroll
    for (int v = 0; v < TV; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (sp_pos(v, e) < n) {
          tm = max(tm, kr[4 * v + e]);
          has = 1;
        }
    for (int i = tid; i < kSplitBins; i += NT) hist[i] = 0;
    __syncthreads();
    if (has) atomicAdd(&hist[tm >> (32 - kSplitBits)], 1u);
    __syncthreads();
    for (int i = tid; i < kSplitBins; i += NT)
      if (hist[i] != 0u) dev_add(rhist + i, hist[i]);
    row_barrier(ctl, phase++, spans);
    // Thread t owns bins 2047-2t and 2046-2t (descending); the k-th
    // largest thread maximum's bin starts the window, the highest
    // non-empty bin ends it.
    const int b0 = kSplitBins - 1 - 2 * tid, b1 = b0 - 1;
    const uint32_t h0 = dev_load(rhist + b0), h1 = dev_load(rhist + b1);
    if (tid == 0) {
      s_bin = -1;
      s_bin_cnt = 0;
    }
    uint32_t tot;
    const uint32_t above = block_exscan<NT>(h0 + h1, tmp, &tot);
    if (above < (uint32_t)keff && (uint32_t)keff <= above + h0) s_bin = b0;
    if (above + h0 < (uint32_t)keff && (uint32_t)keff <= above + h0 + h1) s_bin = b1;
    if (above == 0u && h0 + h1 != 0u) s_bin_cnt = (uint32_t)(h0 != 0u ? b0 : b1);
    __syncthreads();
    const uint32_t top = min(s_bin_cnt, (uint32_t)kSplitBins - 1u);
    const uint32_t lo_edge = s_bin >= 0 ? (uint32_t)s_bin << (32 - kSplitBits) : 0u;
    const uint32_t hi_edge = ((top + 1u) << (32 - kSplitBits)) - 1u;   // (2^32 - 1 wraps to it)
    __syncthreads();

    // 2. Radix passes over the window.
    int lo_fixed = 32 - __clz(lo_edge ^ hi_edge);
    uint32_t prefix = lo_edge;
    need = keff;
    cnt = n;
    int pass = 0;
    // The first pass always runs: it counts each span's keys in the window,
    // which need not be all of them.
    while ((pass == 0 || cnt > (uint32_t)kSmall) && lo_fixed > 0 && pass < kSplitPasses) {
      const int hi = lo_fixed - 1;
      const int lo = hi >= kSplitBits - 1 ? hi - (kSplitBits - 1) : 0;
      const int nb = 1 << (hi - lo + 1);
      for (int i = tid; i < kSplitBins; i += NT) hist[i] = 0;
      __syncthreads();
      const uint32_t fixed_mask = lo_fixed >= 32 ? 0u : (~0u << lo_fixed);
#pragma unroll
      for (int v = 0; v < TV; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = pin(kr[4 * v + e]);
          if (sp_pos(v, e) < n && ((key ^ prefix) & fixed_mask) == 0u)
            atomicAdd(&hist[(key >> lo) & (nb - 1)], 1u);
        }
      __syncthreads();
      uint32_t* rh = rhist + (1 + pass) * kSplitBins;
      for (int i = tid; i < nb; i += NT)
        if (hist[i] != 0u) dev_add(rh + i, hist[i]);
      row_barrier(ctl, phase++, spans);
      // Bins in descending order: thread t owns bins nb-1-2t and nb-2-2t.
      uint32_t g0 = 0, g1 = 0;
      const int c0 = nb - 1 - 2 * tid, c1 = c0 - 1;
      if (c0 >= 0) g0 = dev_load(rh + c0);
      if (c1 >= 0) g1 = dev_load(rh + c1);
      const uint32_t ab = block_exscan<NT>(g0 + g1, tmp, &tot);
      if (c0 >= 0 && ab < need && need <= ab + g0) {
        s_bin = c0;
        s_bin_need = need - ab;
        s_bin_cnt = g0;
      }
      if (c1 >= 0 && ab + g0 < need && need <= ab + g0 + g1) {
        s_bin = c1;
        s_bin_need = need - ab - g0;
        s_bin_cnt = g1;
      }
      __syncthreads();
      const int bin = min(max(s_bin, 0), nb - 1);
      // This span's keys above the chosen bin and in it.
      uint32_t mine = 0;
      if (c0 > bin) mine += hist[c0];
      if (c1 > bin) mine += hist[c1];
      uint32_t my_tot;
      (void)block_exscan<NT>(mine, tmp, &my_tot);
      my_above += my_tot;
      my_inbin = hist[bin];
      prefix = (prefix & ~(uint32_t)(((1ull << (hi + 1)) - 1))) | ((uint32_t)bin << lo);
      need = s_bin_need;
      cnt = s_bin_cnt;
      lo_fixed = lo;
      ++pass;
      __syncthreads();
    }
    bin_lo = ((uint64_t)prefix >> lo_fixed) << lo_fixed;
    win_lo = bin_lo + (1ull << lo_fixed);
  }
  const bool small_bin = !all && cnt <= (uint32_t)kSmall;
  const bool ordered = !all && !small_bin;   // a run of equal keys
  const bool win_any = !all && win_lo <= 0xFFFFFFFFull;
  const uint32_t win32 = (uint32_t)win_lo, bin32 = (uint32_t)bin_lo;

  // 3. Every span's winners, so this span's offset in the winner list.
  uint32_t prefix_g = (uint32_t)min(base, n), my_need = 0;
  uint64_t thr = 0;
  if (!all) {
    if (tid == 0) {
      dev_store(mm + 2 * g, my_above);
      dev_store(mm + 2 * g + 1, my_inbin);
      s_nc = 0;
      s_off = small_bin && my_inbin ? dev_add(ctl + kCtlCand, my_inbin) : 0u;
    }
    if (tid < kSplitMaxSpans) s_win[tid] = 0;
    __syncthreads();
    if (small_bin && my_inbin) {
#pragma unroll
      for (int v = 0; v < TV; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = kr[4 * v + e];
          if (sp_pos(v, e) < n && key >= bin32 && (!win_any || key < win32)) {
            const uint32_t at = s_off + atomicAdd(&s_nc, 1u);
            if (at < (uint32_t)kSmall) dev_store64(gcand + at, full_key(key, sp_pos(v, e)));
          }
        }
    }
    row_barrier(ctl, phase++, spans);
    // Every span's counts, the bin's keys and their number, loaded together.
    uint32_t ab = 0, inb = 0, nc = 0;
    uint64_t cx = 0;
    if (tid < spans) {
      ab = dev_load(mm + 2 * tid);
      inb = dev_load(mm + 2 * tid + 1);
    }
    if (small_bin && tid < 64) {
      cx = dev_load64(gcand + tid);
      nc = min(dev_load(ctl + kCtlCand), (uint32_t)kSmall);
    }
    if (small_bin) {
      // One wave sorts the bin's keys; the best `need` win.
      if (tid < 64) {
        const uint64_t x = wave_bitonic_u64<true>(tid < (int)nc ? cx : 0ull, tid);
        if ((uint32_t)tid == need - 1) s_thr = x;
        if ((uint32_t)tid < need && (uint32_t)tid < nc) {
          const int sp = (int)(~(uint32_t)x) / S;
          if (sp >= 0 && sp < spans) atomicAdd(&s_win[sp], 1u);
        }
      }
      __syncthreads();
    }
    // Per span: winners = keys above the bin + its winners in the bin (a
    // run of equal keys: the first `need` in position order).
    uint32_t t1, wins = 0;
    if (small_bin) {
      if (tid < spans) wins = s_win[tid];
    } else {
      const uint32_t inb_before = block_exscan<NT>(inb, tmp, &t1);
      if (tid < spans) wins = need > inb_before ? min(need - inb_before, inb) : 0u;
    }
    const uint32_t before = block_exscan<NT>(ab + wins, tmp, &t1);
    if (tid == g) {
      s_prefix = before;
      s_need = wins;
    }
    __syncthreads();
    prefix_g = min(s_prefix, (uint32_t)keff);
    my_need = s_need;
    thr = s_thr;
  }

  // 4. This span's winners into the list, in position order: per-thread
  // counts per group of four keys, packed 16 bits each, through a workgroup
  // scan (index order is group-major: v, then thread, then e).
  {
    uint32_t eqr[TV];
#pragma unroll
    for (int v = 0; v < TV; ++v) eqr[v] = my_need;
    // (TV = 4: the four groups' counts fit one 64-bit word, 16 bits each.)
    if (ordered) {
      // Ranks among this span's keys equal to the bin's (index order).
      uint64_t pk = 0, pre, tot;
#pragma unroll
      for (int v = 0; v < TV; ++v) {
        uint64_t ne = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ne += (sp_pos(v, e) < n && kr[4 * v + e] == bin32) ? 1u : 0u;
        pk |= ne << (16 * v);
      }
      pre = block_exscan_u64<NT>(pk, tmp64, &tot);
      uint32_t acc = 0;
#pragma unroll
      for (int v = 0; v < TV; ++v) {
        eqr[v] = acc + (uint32_t)((pre >> (16 * v)) & 0xFFFFu);
        acc += (uint32_t)((tot >> (16 * v)) & 0xFFFFu);
      }
    }
    const uint32_t thr_key = (uint32_t)(thr >> 32), thr_npos = (uint32_t)thr;
    const uint32_t win_mul = win_any ? 1u : 0u;
    uint32_t selm = 0, cv[TV];
    // One loop per case (the cases are uniform over the row).
#define ESS_SPLIT_SEL(TEST)                                                    \
  _Pragma("unroll") for (int v = 0; v < TV; ++v) {                             \
    cv[v] = 0;                                                                 \
    _Pragma("unroll") for (int e = 0; e < 4; ++e) {                            \
      const uint32_t key = pin(kr[4 * v + e]);                                 \
      const uint32_t inr = gt_u32((uint32_t)n, (uint32_t)sp_pos(v, e));        \
      const uint32_t t = inr & (TEST);                                         \
      selm |= t << (4 * v + e);                                                \
      cv[v] += t;                                                              \
    }                                                                          \
  }
    if (all) {
      ESS_SPLIT_SEL(1u)
    } else if (small_bin) {
      ESS_SPLIT_SEL(gt_u32(key, thr_key) |
                    (eq_u32(key, thr_key) & ge_u32(~(uint32_t)sp_pos(v, e), thr_npos)))
    } else {
#pragma unroll
      for (int v = 0; v < TV; ++v) {
        cv[v] = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = pin(kr[4 * v + e]);
          const uint32_t inr = gt_u32((uint32_t)n, (uint32_t)sp_pos(v, e));
          const uint32_t eq = inr & eq_u32(key, bin32);
          const uint32_t t = (inr & win_mul & ge_u32(key, win32)) | (eq & gt_u32(my_need, eqr[v]));
          eqr[v] += eq;
          selm |= t << (4 * v + e);
          cv[v] += t;
        }
      }
    }
#undef ESS_SPLIT_SEL
    uint64_t sk = 0, pre, tot;
#pragma unroll
    for (int v = 0; v < TV; ++v) sk |= (uint64_t)cv[v] << (16 * v);
    pre = block_exscan_u64<NT>(sk, tmp64, &tot);
    uint32_t at = prefix_g;
#pragma unroll
    for (int v = 0; v < TV; ++v) {
      uint32_t o = at + (uint32_t)((pre >> (16 * v)) & 0xFFFFu);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((selm >> (4 * v + e)) & 1u) {
          if (o < (uint32_t)keff) dev_store64(gwin + o, full_key(kr[4 * v + e], sp_pos(v, e)));
          ++o;
        }
      at += (uint32_t)((tot >> (16 * v)) & 0xFFFFu);
    }
  }
#undef sp_pos

  // 5. The last span of the row to finish ranks the list.
  wait_own_memory();
  __syncthreads();
  if (tid == 0) s_last = dev_add(ctl + kCtlDone, 1u) == (uint32_t)spans - 1 ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  const size_t o = ((size_t)b * a.n_tok + j) * k;
  int32_t* op = a.sel_pos + o;
  int32_t* os = a.sel_slot + o;
  // The list, checked: every entry a visible position (anything else means
  // the exchange went wrong, and the row is reported broken).
  uint64_t* pw = dyn + a.kpow2;
  if (tid == 0) s_nc = 0;
  __syncthreads();
  uint32_t lmn = 0xFFFFFFFFu, lmx = 0u;   // the winners' key range
  for (int i = tid; i < keff; i += NT) {
    const uint64_t x = dev_load64(gwin + i);
    const uint32_t p = ~(uint32_t)x;
    if (p >= (uint32_t)n) s_nc = 1;
    lmn = min(lmn, (uint32_t)(x >> 32));
    lmx = max(lmx, (uint32_t)(x >> 32));
    pw[i] = x;
  }
  block_minmax<NT>(lmn, lmx, tmp);
  const bool broken = s_nc != 0u || dev_load(ctl + kCtlBroken) != 0u;
  const int kout = broken ? 0 : keff;
  for (int i = kout + tid; i < k; i += NT) {
    op[i] = -1;
    os[i] = -1;
  }
  if (tid == 0 && a.n_sel) a.n_sel[b * a.n_tok + j] = kout;
  if (broken) {
    if (FUSE && tid == 0) pool::hdr_of(pa.lru, pa.stride, b)->err = 3;
    return;
  }
  if (keff == 0) return;
  int32_t* rpos = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(dyn) + a.rank_off);
  int32_t* rslot = rpos + k;
  const bool lists = !FUSE && a.pl.pos != nullptr;
  const RowOut out{op, os, a.cache_slots + (size_t)b * L, nullptr, nullptr, nullptr,
                   rpos, rslot, pw, lists ? a.pl.pos + o : nullptr,
                   lists ? a.pl.rank + o : nullptr, lists ? a.pl.slot + o : nullptr};
  rank_compact<FUSE, true>(out, keff, a.kpow2, lmx, lmn, dyn, hist, tmp);
  if constexpr (FUSE) {
    __syncthreads();   // selections complete; the sort buffer is free
    pool::update_request<true, true>(pa, b, dyn, rpos, rslot, keff, pw);
  }
}

// Dynamic LDS of the rank-order-by-list path: the scatter buffer (kpow2
// words), then the winners in position order (kpow2 words), one dump word
// per thread for the keys that are not winners, and the input-order index
// of each scattered winner (kpow2 32-bit words).
size_t rank_lds_bytes(int kpow2) {
  return (size_t)(2 * kpow2 + NT) * sizeof(uint64_t) + (size_t)kpow2 * sizeof(uint32_t);
}

// Levels a row of L entries needs before one workgroup holds its candidate
// list (0: the row fits one register-resident chunk, or k is too large for
// levels to shrink the row).
int n_levels(int L, int k) {
  if (k > kLevelMaxK || L <= CHUNK) return 0;
  int nl = 1;
  for (int n = level_count(L, k, 1); n > CHUNK_E; n = level_count(n, k, nl)) ++nl;
  return nl;
}

size_t level_cap(int L, int k) { return (size_t)((L + CHUNK_E - 1) / CHUNK_E) * k; }

size_t level_half(size_t rows, size_t cap) { return align_up(rows * cap * 4, 256); }

// Spans of a split row, and whether a launch of the split selection fits:
// rows over one register chunk, k ranked by sort, and at most half the
// device's compute units' worth of workgroups (every workgroup of a row
// must be resident at once; two launches in flight together still fit).
int split_spans(int L) { return (L + CHUNK_E - 1) / CHUNK_E; }

bool split_shape(const ess_dims& d, int k) {
  const int kpow2 = pow2_at_least(k) < NT ? NT : pow2_at_least(k);
  return d.ctx_len > CHUNK && k <= kFusedMaxK && kpow2 <= kSortRankMax &&
         split_spans(d.ctx_len) <= kSplitMaxSpans;
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cus[dev] = c;
  }
  return cus[dev];
}

bool split_fits(const ess_dims& d, int k, int n_tok) {
  if (!split_shape(d, k)) return false;
  const long wgs = (long)split_spans(d.ctx_len) * d.batch * n_tok;
  return wgs <= device_cus() / 2;
}

size_t split_ws_bytes(const ess_dims& d, int k, int n_tok) {
  if (!split_shape(d, k)) return 0;
  return (size_t)d.batch * n_tok * split_layout(split_spans(d.ctx_len), k).row_bytes;
}

// Clear the rows' control words and pass histograms, then launch the split
// selection (FUSE: with the residency update).
template <bool FUSE>
hipError_t enqueue_split(const ess_dims& d, int k, int n_tok, const float* scores,
                         const int32_t* n_vis, const int32_t* cache_slots,
                         int32_t* sel_pos, int32_t* sel_slot, int32_t* n_sel,
                         void* ws, PosLists pl, const pool::Args& pa, size_t lds,
                         int rank_off, bool cleared, hipStream_t s) {
  const int spans = split_spans(d.ctx_len), rows = d.batch * n_tok;
  const int kpow2 = pow2_at_least(k) < NT ? NT : pow2_at_least(k);
  const SplitLayout lay = split_layout(spans, k);
  hipError_t e = ensure_dyn_lds((const void*)topk_split_kernel<FUSE>, (int)lds);
  if (e != hipSuccess) return e;
  if (!cleared) {
    hipLaunchKernelGGL(split_clear_kernel, dim3(8, rows), dim3(256), 0, s,
                       static_cast<char*>(ws), lay.row_bytes, (int)lay.clear_words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const SplitArgs a{scores, n_vis, cache_slots, sel_pos, sel_slot, n_sel,
                    static_cast<char*>(ws), lay.row_bytes, lay, pl, d.ctx_len, d.mtp,
                    n_tok, k, kpow2, rank_off};
  hipLaunchKernelGGL(topk_split_kernel<FUSE>, dim3(spans, rows), dim3(NT), lds, s, a, pa);
  return hipGetLastError();
}

// Enqueue the levels of every row; *key, *pos: the list the final
// selection reads.
hipError_t enqueue_levels(const ess_dims& d, int k, int n_tok, int nl,
                          const float* scores, const int32_t* n_vis, void* ws,
                          const uint32_t** fkey, const int32_t** fpos,
                          hipStream_t s) {
  const size_t cap = level_cap(d.ctx_len, k);
  const int rows = d.batch * n_tok;
  const size_t half = level_half(rows, cap);
  char* w = static_cast<char*>(ws);
  uint32_t* key[2] = {reinterpret_cast<uint32_t*>(w), reinterpret_cast<uint32_t*>(w + 2 * half)};
  int32_t* pos[2] = {reinterpret_cast<int32_t*>(w + half), reinterpret_cast<int32_t*>(w + 3 * half)};
  int n = d.ctx_len;
  const int kpow2 = pow2_at_least(k) < NT ? NT : pow2_at_least(k);
  for (int l = 1; l <= nl; ++l) {
    const int chunks = (n + level_chunk(l) - 1) / level_chunk(l);
    const int ob = (l - 1) & 1, ib = ob ^ 1;
    if (l == 1)
      hipLaunchKernelGGL(topk_level_kernel<false>, dim3(chunks, rows), dim3(NT), 0, s,
                         scores, n_vis, nullptr, nullptr, key[ob], pos[ob], cap,
                         d.ctx_len, d.mtp, n_tok, k, kpow2, l);
    else
      hipLaunchKernelGGL(topk_level_kernel<true>, dim3(chunks, rows), dim3(NT), 0, s,
                         scores, n_vis, key[ib], pos[ib], key[ob], pos[ob], cap,
                         d.ctx_len, d.mtp, n_tok, k, kpow2, l);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    n = level_count(n, k, l);
  }
  *fkey = key[(nl - 1) & 1];
  *fpos = pos[(nl - 1) & 1];
  return hipSuccess;
}

}  // namespace

size_t topk_ws_bytes(const ess_dims& d, int k, int n_tok) {
  if (n_levels(d.ctx_len, k) == 0) return 0;
  const size_t lv = 4 * level_half((size_t)d.batch * n_tok, level_cap(d.ctx_len, k));
  const size_t sp = split_ws_bytes(d, k, n_tok);
  return lv > sp ? lv : sp;
}

bool topk_pos_lists_fit(const ess_dims& d, int k, bool levels) {
  const int kpow2 = pow2_at_least(k) < NT ? NT : pow2_at_least(k);
  const bool nl = levels && n_levels(d.ctx_len, k) > 0;
  return kpow2 <= kSortRankMax && (d.ctx_len <= CHUNK || nl);
}

bool split_clear(const ess_dims& d, int k, int n_tok, void* ws, ClearSpec* c) {
  if (!ws || n_levels(d.ctx_len, k) == 0 || !split_fits(d, k, n_tok)) return false;
  const SplitLayout lay = split_layout(split_spans(d.ctx_len), k);
  *c = ClearSpec{static_cast<uint32_t*>(ws), lay.row_bytes / 4, (int)lay.clear_words,
                 d.batch * n_tok};
  return true;
}

hipError_t launch_topk(const ess_dims& d, int k, int n_tok,
                       const float* scores, const int32_t* n_vis,
                       const int32_t* cache_slots, int32_t* sel_pos,
                       int32_t* sel_slot, int32_t* n_sel, void* ws,
                       hipStream_t s, PosLists pl, bool cleared, bool split) {
  // The sorts need a power of two of at least one key per thread.  Rows
  // held in registers (and candidate lists) rank their winners by a sort
  // over a second kpow2-word buffer up to kSortRankMax.
  const int kpow2 = pow2_at_least(k) < NT ? NT : pow2_at_least(k);
  const size_t lds1 = (size_t)kpow2 * sizeof(uint64_t);
  const size_t lds2 = kpow2 <= kSortRankMax ? rank_lds_bytes(kpow2) : lds1;
  const int nl = ws ? n_levels(d.ctx_len, k) : 0;
  size_t lds = lds2;
  if (nl > 0 && split && split_fits(d, k, n_tok)) {
    // The position lists' ranks and slots are staged in LDS after the sort
    // buffers, then written in order.
    const size_t roff = align_up(rank_lds_bytes(kpow2), 16);
    return enqueue_split<false>(d, k, n_tok, scores, n_vis, cache_slots, sel_pos,
                                sel_slot, n_sel, ws, pl, pool::Args{},
                                roff + 2 * (size_t)k * sizeof(int32_t), (int)roff, cleared, s);
  }
  if (nl > 0) {
    const uint32_t* fk;
    const int32_t* fp;
    hipError_t e = enqueue_levels(d, k, n_tok, nl, scores, n_vis, ws, &fk, &fp, s);
    if (e != hipSuccess) return e;
    const bool bys = kpow2 <= kSortRankMax;
    const void* ff = bys ? (const void*)topk_final_kernel<true>
                         : (const void*)topk_final_kernel<false>;
    e = ensure_dyn_lds(ff, (int)lds);
    if (e != hipSuccess) return e;
    if (bys)
      hipLaunchKernelGGL(topk_final_kernel<true>, dim3(d.batch * n_tok), dim3(NT), lds, s,
                         fk, fp, level_cap(d.ctx_len, k), n_vis, cache_slots, sel_pos,
                         sel_slot, n_sel, d.ctx_len, d.mtp, n_tok, k, kpow2, nl, pl);
    else
      hipLaunchKernelGGL(topk_final_kernel<false>, dim3(d.batch * n_tok), dim3(NT), lds, s,
                         fk, fp, level_cap(d.ctx_len, k), n_vis, cache_slots, sel_pos,
                         sel_slot, n_sel, d.ctx_len, d.mtp, n_tok, k, kpow2, nl,
                         PosLists{nullptr, nullptr, nullptr});
    return hipGetLastError();
  }
  // Rows of at most one chunk stay in registers for all passes.
  const bool res = d.ctx_len <= CHUNK;
  const bool bys = res && kpow2 <= kSortRankMax;
  lds = bys ? lds2 : lds1;
  const void* fn = bys ? (const void*)topk_kernel<true, true>
                   : res ? (const void*)topk_kernel<true, false>
                         : (const void*)topk_kernel<false, false>;
  hipError_t e = ensure_dyn_lds(fn, (int)lds);
  if (e != hipSuccess) return e;
#define ESS_TOPK_LAUNCH(R, S, PL)                                              \
  hipLaunchKernelGGL((topk_kernel<R, S>), dim3(d.batch * n_tok), dim3(NT), lds, s, \
                     scores, n_vis, cache_slots, sel_pos, sel_slot, n_sel,       \
                     d.ctx_len, d.mtp, n_tok, k, kpow2, PL)
  const PosLists none{nullptr, nullptr, nullptr};
  if (bys)
    ESS_TOPK_LAUNCH(true, true, pl);
  else if (res)
    ESS_TOPK_LAUNCH(true, false, none);
  else
    ESS_TOPK_LAUNCH(false, false, none);
#undef ESS_TOPK_LAUNCH
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
                                void* ws, hipStream_t s, bool cleared, bool split) {
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
  const int nl = ws ? n_levels(d.ctx_len, k) : 0;
  const bool res = d.ctx_len <= CHUNK;
  // Register-resident rows and candidate lists rank by a sort: the sort
  // buffer and the position-ordered winners (the update then sorts
  // nothing); streamed rows use winner buckets and the update sorts.
  const bool sorted = res || nl > 0;
  const size_t topk_bytes = sorted ? rank_lds_bytes(kpow2) : (size_t)kpow2 * sizeof(uint64_t);
  const size_t upd_bytes = sorted ? (size_t)epow2 * sizeof(uint64_t)
                                  : (size_t)epow2 * sizeof(uint64_t) * (two ? 2 : 1);
  const size_t rank_off = align_up(topk_bytes > upd_bytes ? topk_bytes : upd_bytes, 16);
  const size_t lds = rank_off + 2 * (size_t)k * sizeof(int32_t);
  if (nl > 0 && split && split_fits(d, k, 1))
    return enqueue_split<true>(d, k, 1, scores, n_vis, cache_slots, sel_pos, sel_slot,
                               n_sel, ws, PosLists{nullptr, nullptr, nullptr}, pa, lds,
                               (int)rank_off, cleared, s);
  const uint32_t* fk = nullptr;
  const int32_t* fp = nullptr;
  const void* fn = nl > 0 ? (const void*)select_update_kernel<true, true>
                   : res  ? (const void*)select_update_kernel<true, false>
                          : (const void*)select_update_kernel<false, false>;
  hipError_t e = ensure_dyn_lds(fn, (int)lds);
  if (e != hipSuccess) return e;
  if (nl > 0) {
    e = enqueue_levels(d, k, 1, nl, scores, n_vis, ws, &fk, &fp, s);
    if (e != hipSuccess) return e;
  }
  const size_t cap = level_cap(d.ctx_len, k);
#define ESS_SU_LAUNCH(R, X)                                                    \
  hipLaunchKernelGGL((select_update_kernel<R, X>), dim3(d.batch), dim3(NT), lds, s, \
                     scores, fk, fp, cap, n_vis, cache_slots, sel_pos, sel_slot,   \
                     n_sel, d.ctx_len, d.mtp, k, kpow2, nl, pa, (int)rank_off)
  if (nl > 0)
    ESS_SU_LAUNCH(true, true);
  else if (res)
    ESS_SU_LAUNCH(true, false);
  else
    ESS_SU_LAUNCH(false, false);
#undef ESS_SU_LAUNCH
  return hipGetLastError();
}

}  // namespace ess
