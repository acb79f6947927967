// Offline replay of the hot pool under an eviction policy (host code).
//
// The pages compare eviction policies by recording the per-step top-k index
// sets of a run and replaying them offline through a pool simulator,
// changing only the policy (FlashOffloading analysis, decode ablation, first
// group, and Fig. 8: Random, LRU, Score, LIM; capacity matters more than
// policy).  This is that simulator for the pool of this library: the same
// first fill, misses = union of the step's ways minus the residents, free
// slots first, then one victim per remaining miss among the residents
// outside the union, chosen by the policy:
//   LRU    - smallest (last step in a union, position): the pool's own order
//            (within a step, and the fill, positions become recent in
//            ascending order);
//   Score  - smallest (the step's score, position), a position's score being
//            the largest of its index scores over the step's ways;
//   Random - smallest (key, position), the key being output number
//            (request << 48 | step << 32 | position) + 1 of the SplitMix64
//            generator (Steele, Lea and Flood, OOPSLA 2014) seeded with seed.
// Only counts are kept: which slot a miss takes does not change the counts.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <utility>
#include <vector>

#include "ess.h"
#include "ess_host.h"

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

uint64_t splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t random_key(uint64_t seed, uint64_t request, uint64_t step, uint64_t pos) {
  const uint64_t counter = (request << 48) | (step << 32) | pos;
  return splitmix64_mix(seed + (counter + 1) * kGamma);
}

}  // namespace

extern "C" ess_status ess_replay_evictions(
    int32_t policy, int32_t ctx_len, int32_t pool_slots, int32_t steps,
    int32_t mtp, int32_t topk, const float* scores, const int32_t* sel_pos,
    const int32_t* n_sel, uint64_t seed, int32_t request, int32_t* n_miss,
    int32_t* n_evict) {
  const char* fn = "ess_replay_evictions";
  if (policy != ESS_EVICT_LRU && policy != ESS_EVICT_RANDOM &&
      policy != ESS_EVICT_SCORE)
    return ess::host_fail(ESS_ERR_INVALID, "%s: unknown policy %d", fn, policy);
  if (ctx_len < 1 || pool_slots < 1 || steps < 1 || steps > 0xFFFF ||
      mtp < 1 || topk < 1 || request < 0 || request > 0xFFFF)
    return ess::host_fail(ESS_ERR_INVALID,
                         "%s: bad sizes (ctx_len %d, pool_slots %d, steps %d, "
                         "mtp %d, topk %d, request %d)",
                         fn, ctx_len, pool_slots, steps, mtp, topk, request);
  if (!scores || !sel_pos || !n_sel || !n_miss)
    return ess::host_fail(ESS_ERR_INVALID, "%s: NULL array", fn);

  const size_t L = (size_t)ctx_len;
  const int64_t C = pool_slots;
  auto score = [&](int t, int j, size_t p) {
    return scores[((size_t)t * mtp + j) * L + p];
  };

  std::vector<uint8_t> res(L, 0);          // resident?
  std::vector<int32_t> last(L, -2);        // last step in a union (fill: -1)
  std::vector<int32_t> mark(L, -1);        // step whose union holds it
  std::vector<int32_t> where(L, -1);       // index in `live`
  std::vector<int32_t> live;               // resident positions
  live.reserve((size_t)C);

  // First fill: top-min(C, visible) of way 0 at step 0, score descending,
  // position ascending.
  {
    std::vector<int32_t> vis;
    for (size_t p = 0; p < L; ++p)
      if (std::isfinite(score(0, 0, p))) vis.push_back((int32_t)p);
    const size_t n = std::min<size_t>((size_t)C, vis.size());
    auto better = [&](int32_t a, int32_t b) {
      const float sa = score(0, 0, a), sb = score(0, 0, b);
      return sa > sb || (sa == sb && a < b);
    };
    if (n < vis.size()) std::nth_element(vis.begin(), vis.begin() + n, vis.end(), better);
    for (size_t i = 0; i < n; ++i) {
      const int32_t p = vis[i];
      res[p] = 1;
      last[p] = -1;
      where[p] = (int32_t)live.size();
      live.push_back(p);
    }
  }
  int64_t free_slots = C - (int64_t)live.size();

  std::vector<int32_t> uni;
  std::vector<std::pair<uint64_t, int32_t>> cand_u;   // (key, position)
  std::vector<std::pair<float, int32_t>> cand_f;
  for (int t = 0; t < steps; ++t) {
    uni.clear();
    for (int j = 0; j < mtp; ++j) {
      const int n = std::min(std::max(n_sel[(size_t)t * mtp + j], 0), topk);
      const int32_t* row = sel_pos + ((size_t)t * mtp + j) * topk;
      for (int i = 0; i < n; ++i) {
        const int32_t p = row[i];
        if (p < 0 || (size_t)p >= L)
          return ess::host_fail(ESS_ERR_INVALID, "%s: position %d out of range at step %d",
                               fn, p, t);
        if (mark[p] != t) {
          mark[p] = t;
          uni.push_back(p);
        }
      }
    }
    if ((int64_t)uni.size() > C)
      return ess::host_fail(ESS_ERR_CAPACITY, "%s: union of %zu exceeds %d slots at step %d",
                           fn, uni.size(), pool_slots, t);
    int64_t misses = 0;
    for (int32_t p : uni) misses += res[p] ? 0 : 1;
    const int64_t from_free = std::min(free_slots, misses);
    free_slots -= from_free;
    const int64_t need = misses - from_free;

    if (need > 0) {
      // Residents outside the union, ordered by the policy's key; the
      // first `need` are the victims.
      std::vector<int32_t> victims;
      if (policy == ESS_EVICT_SCORE) {
        cand_f.clear();
        for (int32_t p : live) {
          if (mark[p] == t) continue;
          float best = score(t, 0, (size_t)p);
          for (int j = 1; j < mtp; ++j) best = std::max(best, score(t, j, (size_t)p));
          cand_f.emplace_back(best, p);
        }
        std::nth_element(cand_f.begin(), cand_f.begin() + (need - 1), cand_f.end());
        for (int64_t i = 0; i < need; ++i) victims.push_back(cand_f[i].second);
      } else {
        cand_u.clear();
        for (int32_t p : live) {
          if (mark[p] == t) continue;
          const uint64_t key =
              policy == ESS_EVICT_LRU
                  ? (uint64_t)((int64_t)last[p] + 2)        // -1 (fill) -> 1
                  : random_key(seed, (uint64_t)request, (uint64_t)t, (uint64_t)p);
          cand_u.emplace_back(key, p);
        }
        std::nth_element(cand_u.begin(), cand_u.begin() + (need - 1), cand_u.end());
        for (int64_t i = 0; i < need; ++i) victims.push_back(cand_u[i].second);
      }
      for (int32_t p : victims) {
        res[p] = 0;
        const int32_t w = where[p], tail = live.back();
        live[w] = tail;
        where[tail] = w;
        live.pop_back();
        where[p] = -1;
      }
    }
    for (int32_t p : uni) {
      if (!res[p]) {
        res[p] = 1;
        where[p] = (int32_t)live.size();
        live.push_back(p);
      }
      last[p] = t;
    }
    n_miss[t] = (int32_t)misses;
    if (n_evict) n_evict[t] = (int32_t)need;
  }
  return ESS_OK;
}
