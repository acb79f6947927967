// Residency update of one request, shared by the standalone pool-update
// kernel and the fused select-and-update kernel.  See pool_update.hip for
// the method.
#pragma once

#include "block_util.h"
#include "ess_internal.h"

namespace ess {
namespace pool {

constexpr int NT = 1024;
constexpr int kSortBuckets = 2048;
constexpr int kTwoBufferMax = 4096;   // entries sorted out of place up to this

struct Ring {
  int32_t slot;
  int32_t stamp;
};

__device__ __forceinline__ LruHeader* hdr_of(void* lru, size_t stride, int b) {
  return reinterpret_cast<LruHeader*>(static_cast<char*>(lru) + stride * b);
}

// Entry layout (64 bits, sorted ascending): position (28 bits) | token (2) |
// row (14) | slot + 1 (20; a hit's slot from the start, 0 for a miss until
// it is paired).  Sorting on the whole value orders positions ascending
// and, for a repeated position, the smallest token first (the entries of a
// position carry the same slot); a miss's run head gets its slot in place
// once paired, so every row's outputs come from LDS.
__device__ __forceinline__ uint64_t make_entry(int pos, int j, int i) {
  return ((uint64_t)(uint32_t)pos << 36) | ((uint64_t)j << 34) | ((uint64_t)i << 20);
}
__device__ __forceinline__ int ent_pos(uint64_t e) { return (int)(e >> 36); }
__device__ __forceinline__ int ent_tok(uint64_t e) { return (int)((e >> 34) & 3); }
__device__ __forceinline__ int ent_row(uint64_t e) { return (int)((e >> 20) & 0x3FFF); }
__device__ __forceinline__ int ent_slot(uint64_t e) { return (int)(e & 0xFFFFF) - 1; }
__device__ __forceinline__ uint64_t with_slot(uint64_t e, int slot) {
  return (e & ~0xFFFFFull) | (uint64_t)(slot + 1);
}
constexpr uint64_t kNoEntry = ~0ull;

struct Args {
  const int32_t* sel_pos;
  const int32_t* n_sel;
  int32_t* cache_slots;
  int32_t* slot_pos;
  void* lru;
  size_t stride;
  int32_t* miss_pos;
  int32_t* miss_slot;
  int32_t* n_miss_out;
  int32_t* n_evict_out;
  int32_t* row_dst;
  int32_t* sel_slot_post;
  int L, C, k, n_tok, epow2, two_buffers, pos_shift;
  // Optional: every row's slot before this update as the top-k read it
  // (cache_slots at sel_pos); read next to sel_pos instead of looking
  // cache_slots up at each position after sel_pos arrives.
  const int32_t* sel_slot_pre;
  // Optional (MERGE): each token's selection in ascending position order
  // with its rank and slot, from the top-k.
  PosLists lists;
};

// The update of request b by a 1024-thread workgroup.  smem_ent: epow2
// entries of LDS (twice that when two_buffers).  PRESEL: one query token
// whose n_pre selected positions and their cache_slots values (read before
// this update) are already in LDS (pre_pos, pre_slot); otherwise the
// selections of every token are read from sel_pos / n_sel.  SORTED (with
// PRESEL): the selection is already in ascending position order in LDS -
// pw[i] holds entry i's full selection key (its low word ~position),
// pre_pos[i] its rank and pre_slot[i] its slot - so the entries are built
// in order and not sorted.
//   MERGE (without PRESEL): every token's selection comes in ascending
// position order (a.lists); the entries are placed by merging those lists
// (each entry's place: its index in its own list plus, for every other
// token, the entries before it there - equal positions: smaller token
// first), so nothing is sorted.  Needs a second epow2-entry LDS buffer.
template <bool PRESEL, bool SORTED = false, bool MERGE = false>
__device__ __forceinline__ void update_request(const Args& a, int b, uint64_t* smem_ent,
                               const int32_t* pre_pos, const int32_t* pre_slot,
                               int n_pre, const uint64_t* pw = nullptr) {
  static_assert(!SORTED || PRESEL, "a sorted selection comes from the fused top-k");
  static_assert(!MERGE || !PRESEL, "merged lists come from the top-k's outputs");
  __shared__ uint32_t tmp[NT / 64 + 1];
  __shared__ uint64_t tmp64[NT / 64 + 1];
  __shared__ uint32_t bcnt[kSortBuckets];
  __shared__ uint32_t rc[4 * 64 + 1];   // ring compaction: (row, wave) counts, then places
  __shared__ int s_head_new;
  uint64_t* ent = smem_ent;
  const int L = a.L, C = a.C, k = a.k, n_tok = a.n_tok, epow2 = a.epow2;
  const int32_t* sel_pos = a.sel_pos;
  int32_t* miss_pos = a.miss_pos;
  int32_t* miss_slot = a.miss_slot;
  int32_t* row_dst = a.row_dst;
  int32_t* sel_slot_post = a.sel_slot_post;
  const int tid = threadIdx.x;
  LruHeader* h = hdr_of(a.lru, a.stride, b);
  int32_t* stamp = reinterpret_cast<int32_t*>(h + 1);
  Ring* ring = reinterpret_cast<Ring*>(stamp + C);
  int32_t* cs = a.cache_slots + (size_t)b * L;
  int32_t* sp = a.slot_pos + (size_t)b * C;
  const size_t list0 = (size_t)b * n_tok * k;   // copy-list base
  const size_t rows0 = (size_t)b * n_tok * k;   // per-row arrays base

  const int head0 = h->head, tail0 = h->tail, free_head = h->free_head;
  const int epoch = h->epoch, cap = h->cap;

  int off[5];
  off[0] = 0;
  if (PRESEL) {
    off[1] = n_pre;
  } else {
    for (int j = 0; j < n_tok; ++j)
      off[j + 1] = off[j] + min(max(a.n_sel[b * n_tok + j], 0), k);
  }
  const int n_e = off[n_tok];

  // 0. Row outputs start empty.
  for (int i = tid; i < n_tok * k; i += NT) {
    row_dst[rows0 + i] = -1;
    sel_slot_post[rows0 + i] = -1;
  }
  // 1. Entries of every way, each with its position's slot before this
  // update (the selection's own lookup, or cache_slots: every thread's reads
  // are independent and in flight together), then sort.  Out-of-range
  // positions are dropped (they sort last and end the scan).
  bool bad = false;
  constexpr int kU = 4;   // entries per thread whose reads are in flight together
  if constexpr (MERGE) {
    // Every entry's position, rank and slot are read first, all of a
    // thread's reads in flight together (the merge runs with two buffers,
    // so n_e <= kTwoBufferMax = kU * NT).  Two tokens: a merge path.  More:
    // the positions go to the second buffer, then each entry finds its
    // merged place by binary searches in the other tokens' lists.
    static_assert(kTwoBufferMax <= kU * NT, "one read per entry slot below");
    int32_t* lp = reinterpret_cast<int32_t*>(smem_ent + epow2);
    int pos[kU], rk[kU], sl[kU], tok[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = tid + u * NT;
      pos[u] = -1;
      rk[u] = 0;
      sl[u] = -1;
      tok[u] = 0;
      if (e < n_e) {
        int j = 0;
        while (e >= off[j + 1]) ++j;
        const size_t li = rows0 + (size_t)j * k + (e - off[j]);
        tok[u] = j;
        pos[u] = a.lists.pos[li];
        rk[u] = a.lists.rank[li];
        sl[u] = a.lists.slot[li];
      }
    }
    if (n_tok == 2) {
      // Two lists: a merge path.  Every entry's whole key goes to the second
      // buffer at its list index (list 0 then list 1, each ascending; a
      // position both tokens selected orders token 0 first, as the keys
      // do, and keys are unique).  Thread t then finds, by one binary
      // search along the diagonal d = 4 t, how many of the first d merged
      // entries come from list 0, and writes merged entries d .. d + 3.
      // An out-of-range position (never from the top-k) is flagged and
      // its key sorts last.
      uint64_t* lk = smem_ent + epow2;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int e = tid + u * NT;
        if (e >= n_e) continue;
        uint64_t key = kNoEntry;
        if (pos[u] >= 0 && pos[u] < L) {
          key = make_entry(pos[u], tok[u], rk[u]);
          if (sl[u] >= 0 && sl[u] < C) key = with_slot(key, sl[u]);
        } else {
          bad = true;
        }
        lk[e] = key;
      }
      for (int e = tid; e < epow2; e += NT) ent[e] = kNoEntry;   // places past n_e
      __syncthreads();
      const int nA = off[1], nB = off[2] - off[1];
      const uint64_t* A = lk;
      const uint64_t* B = lk + nA;
      const int d0 = tid * kU;
      if (d0 < n_e) {
        int lo = max(0, d0 - nB), hi = min(d0, nA);
        while (lo < hi) {   // A[mid] among the first d0 <=> it precedes B[d0 - mid - 1]
          const int mid = (lo + hi) >> 1;
          if (A[mid] < B[d0 - mid - 1]) lo = mid + 1;
          else hi = mid;
        }
        int i = lo, j = d0 - lo;
#pragma unroll
        for (int q = 0; q < kU; ++q) {
          if (d0 + q >= n_e) break;
          const bool from_a = i < nA && (j >= nB || A[i] < B[j]);
          ent[d0 + q] = from_a ? A[i++] : B[j++];
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int e = tid + u * NT;
        if (e < n_e) lp[e] = pos[u];
      }
      // (every place starts empty: an entry that could not be placed leaves
      // a kNoEntry, which ends the scans below, never a stale entry)
      for (int e = tid; e < epow2; e += NT) ent[e] = kNoEntry;
      __syncthreads();
      // Place = index in its own list + the entries before it in every other
      // list (positions below it, and its own position when that list's token
      // is smaller).  Round d searches list (token + d) mod n_tok for each of
      // a thread's entries, in lockstep with the same power-of-two steps
      // (uniform over the workgroup, sized for the longest list), so their
      // LDS reads are in flight together.
      int at[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) at[u] = tid + u * NT - off[tok[u]];
      int len_max = 0;
      for (int j = 0; j < n_tok; ++j) len_max = max(len_max, off[j + 1] - off[j]);
      // steps S, S/2, ..., 1 reach up to index 2S - 2 >= len_max - 1
      const int s0 = pow2_at_least_dev((uint32_t)len_max + 1u) >> 1;
      for (int d = 1; d < n_tok; ++d) {
        const int32_t* l2[kU];
        int len[kU], last[kU];
        bool before[kU];                      // equal positions of list j2 come first
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          int j2 = tok[u] + d;
          if (j2 >= n_tok) j2 -= n_tok;
          l2[u] = lp + off[j2];
          len[u] = off[j2 + 1] - off[j2];
          before[u] = j2 < tok[u];
          last[u] = -1;
        }
        for (int step = s0; step >= 1; step >>= 1) {
          // Every load is made (at a clamped index inside the list region),
          // so none waits behind a branch; a probe past the list's end
          // compares as above every position.
          int32_t v[kU];
#pragma unroll
          for (int u = 0; u < kU; ++u)
            v[u] = l2[u][min(last[u] + step, max(len[u] - 1, 0))];
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const int cand = last[u] + step;
            const bool take = (cand < len[u]) & ((v[u] < pos[u]) | (before[u] & (v[u] == pos[u])));
            last[u] = take ? cand : last[u];
          }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) at[u] += last[u] + 1;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int e = tid + u * NT;
        if (e >= n_e) break;
        const int p = pos[u];
        if (p < 0 || p >= L) {                // cannot come from the top-k
          bad = true;
          continue;
        }
        uint64_t key = make_entry(p, tok[u], rk[u]);
        if (sl[u] >= 0 && sl[u] < C) key = with_slot(key, sl[u]);
        ent[min(at[u], n_e - 1)] = key;
      }
    }
  } else if constexpr (SORTED) {
    // Positions come from the selection over [0, n_vis), so all are valid
    // (an invalid one would end the list here, flagged).
    for (int e = tid; e < epow2; e += NT) {
      uint64_t key = kNoEntry;
      if (e < n_e) {
        const int pos = (int)(~(uint32_t)pw[e]);
        if (pos >= 0 && pos < L) {
          key = make_entry(pos, 0, pre_pos[e]);
          const int sl = pre_slot[e];
          if (sl >= 0 && sl < C) key = with_slot(key, sl);
        } else {
          bad = true;
        }
      }
      ent[e] = key;
    }
  } else
  for (int eb = tid; eb < epow2; eb += kU * NT) {
    int pos[kU], row[kU], tok[kU], slot[kU], given[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = eb + u * NT;
      pos[u] = -1;
      row[u] = 0;
      tok[u] = 0;
      given[u] = -1;
      if (e < n_e) {
        int j = 0;
        while (e >= off[j + 1]) ++j;
        tok[u] = j;
        row[u] = e - off[j];
        pos[u] = PRESEL ? pre_pos[row[u]] : sel_pos[rows0 + (size_t)j * k + row[u]];
        if (!PRESEL && a.sel_slot_pre)
          given[u] = a.sel_slot_pre[rows0 + (size_t)j * k + row[u]];
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      slot[u] = pos[u] >= 0 && pos[u] < L
                    ? (PRESEL ? pre_slot[row[u]] : a.sel_slot_pre ? given[u] : cs[pos[u]])
                    : -1;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = eb + u * NT;
      if (e >= epow2) break;
      uint64_t key = kNoEntry;
      if (e < n_e) {
        if (pos[u] >= 0 && pos[u] < L) {
          key = make_entry(pos[u], tok[u], row[u]);
          if (slot[u] >= 0 && slot[u] < C) key = with_slot(key, slot[u]);
        } else {
          bad = true;
        }
      }
      ent[e] = key;
    }
  }
  if (bad) h->err = 2;
  __syncthreads();
  // Sort by position: buckets of the position's top 11 bits (selections are
  // spread over the context, so buckets hold a few entries each), ordered
  // within a bucket on the whole entry; a full sort if the buckets come out
  // uneven or there is no room for a second buffer.
  if (!SORTED && !MERGE) {
    bool done = false;
    if (a.two_buffers) {
      const int shift = a.pos_shift;
      auto bucket = [&](uint64_t x) {
        const int bk = ent_pos(x) >> shift;
        return bk < kSortBuckets ? bk : kSortBuckets - 1;   // dropped entries last
      };
      done = bucket_sort_u64<NT, false>(smem_ent, smem_ent + epow2, n_e, kSortBuckets,
                                        bucket, bcnt, tmp, 256);
    }
    if (!done) block_sort_u64_n<NT, false>(smem_ent, epow2);
  }

  // 2. Unique positions (first entry of each run): a hit's stamp moves to
  // this update (its old ring entry dies).
  const int per = (epow2 + NT - 1) / NT;       // entries per thread, contiguous
  const int e0 = tid * per;
  auto head_of_run = [&](int e) {
    return e == 0 || ent_pos(ent[e - 1]) != ent_pos(ent[e]);
  };
  uint32_t n_u_mine = 0, n_m_mine = 0;
  for (int q = 0; q < per; ++q) {
    const int e = e0 + q;
    if (e >= n_e || ent[e] == kNoEntry) break;
    if (head_of_run(e)) {
      ++n_u_mine;
      const int slot = ent_slot(ent[e]);
      if (slot >= 0) stamp[slot] = epoch;
      else ++n_m_mine;
    }
  }
  // Both counts in one scan: unique positions in the low half, misses in
  // the high half (each total is at most n_e, so neither half carries).
  uint64_t um_tot;
  const uint64_t um_base =
      block_exscan_u64<NT>(((uint64_t)n_m_mine << 32) | n_u_mine, tmp64, &um_tot);
  const uint32_t u_base = (uint32_t)um_base, m_base = (uint32_t)(um_base >> 32);
  const uint32_t n_u = (uint32_t)um_tot, n_miss = (uint32_t)(um_tot >> 32);

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
      if (e >= n_e || ent[e] == kNoEntry) break;
      if (!head_of_run(e) || ent_slot(ent[e]) >= 0) continue;   // hit
      const int pos = ent_pos(ent[e]);
      const int v = (int)mi < use_free ? free_head + (int)mi
                                       : miss_slot[list0 + mi];
      if ((int)mi < paired && v >= 0 && v < C) {
        cs[pos] = v;
        sp[v] = pos;
        stamp[v] = epoch;
        miss_pos[list0 + mi] = pos;
        miss_slot[list0 + mi] = v;
        row_dst[rows0 + (size_t)ent_tok(ent[e]) * k + ent_row(ent[e])] = v;
        ent[e] = with_slot(ent[e], v);
      }
      ++mi;
    }
  }
  __syncthreads();

  // 5. Make room on the ring: compact live entries to the front in order.
  // A round takes kC rows of NT consecutive entries (entry src + q NT + t
  // to thread t, so every read is coalesced), with all of a thread's ring
  // reads and then its stamp reads in flight together: a 4C ring is a few
  // rounds, not 4C / NT rounds of two memory round trips each.  An entry's
  // place: the live entries of the round's earlier rows, of the earlier
  // waves in its row (per-wave counts from ballots, scanned in (row, wave)
  // order by one wave) and of the earlier lanes of its wave.  A round reads
  // all of its entries before it writes any (a barrier between), and it
  // writes only below the next round's start: dst counts the live entries
  // of the earlier rounds, so dst <= src, and a round has at most NT kC live
  // entries.  No entry is overwritten before it is read.
  int tail = tail0;
  if (tail + (int)n_u > cap) {
    constexpr int kC = 16;
    constexpr int kWaves = NT / 64;
    static_assert(kC * kWaves == 4 * 64, "one wave scans the (row, wave) counts, four each");
    const int lane = tid & 63, wv = tid >> 6;
    int dst = 0;
    for (int src = head; src < tail; src += NT * kC) {
      Ring r[kC];
#pragma unroll
      for (int q = 0; q < kC; ++q) {
        const int idx = src + q * NT + tid;
        r[q] = idx < tail ? ring[idx] : Ring{-1, 0};
      }
      int32_t st[kC];
#pragma unroll
      for (int q = 0; q < kC; ++q)
        st[q] = r[q].slot >= 0 && r[q].slot < C ? stamp[r[q].slot] : 0;
      uint32_t live = 0, below[kC];
#pragma unroll
      for (int q = 0; q < kC; ++q) {
        const bool l = r[q].slot >= 0 && r[q].slot < C && st[q] == r[q].stamp;
        const uint64_t bq = __ballot(l);
        below[q] = __builtin_amdgcn_mbcnt_hi((uint32_t)(bq >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bq, 0u));
        if (lane == 0) rc[q * kWaves + wv] = (uint32_t)__popcll(bq);
        live |= (l ? 1u : 0u) << q;
      }
      __syncthreads();
      if (wv == 0) {
        uint32_t c4[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c4[j] = rc[lane * 4 + j];
          sum += c4[j];
        }
        const uint32_t incl = wave_incl_sum(sum);
        uint32_t run = incl - sum;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          rc[lane * 4 + j] = run;
          run += c4[j];
        }
        if (lane == 63) rc[kC * kWaves] = incl;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kC; ++q)
        if ((live >> q) & 1u) ring[dst + (int)rc[q * kWaves + wv] + (int)below[q]] = r[q];
      dst += (int)rc[kC * kWaves];
      __syncthreads();
    }
    head = 0;
    tail = dst;
    if (tid == 0) h->compactions += 1;
  }

  // 6. Push the union in ascending position order with current slots, and
  // every row's slot after the update (from its run's first entry, at most
  // n_tok - 1 entries back).
  for (int q = 0, u = (int)u_base; q < per; ++q) {
    const int e = e0 + q;
    if (e >= n_e || ent[e] == kNoEntry) break;
    const uint64_t x = ent[e];
    int hd = e;
    while (hd > 0 && ent_pos(ent[hd - 1]) == ent_pos(x)) --hd;
    const int slot = ent_slot(ent[hd]);
    sel_slot_post[rows0 + (size_t)ent_tok(x) * k + ent_row(x)] = slot;
    if (hd == e) {
      Ring r;
      r.slot = slot;
      r.stamp = epoch;
      ring[tail + u] = r;
      ++u;
    }
  }
  if (tid == 0) {
    h->head = head;
    h->tail = tail + (int)n_u;
    h->free_head = free_head + use_free;
    h->epoch = epoch + 1;
    // A dry victim scan (flagged) leaves misses unpaired: the copy list and
    // the counts hold the paired ones only.
    a.n_miss_out[b] = use_free + found;
    a.n_evict_out[b] = found;
  }
}


}  // namespace pool
}  // namespace ess
