// Workgroup-wide helpers: scans, reductions and an LDS bitonic sort.
// Every helper must be reached by all threads of the workgroup.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ess {

// Smallest power of two >= x (1 for x <= 1).
__device__ __forceinline__ int pow2_at_least_dev(uint32_t x) {
  return x <= 1u ? 1 : (int)(1u << (32 - __clz(x - 1u)));
}

// Inclusive scans over the 64 lanes of a wave in registers, with gfx9's
// DPP lane moves: row_shr 1, 2, 4, 8 within each row of 16 lanes, then
// row_bcast:15 (the last lane of rows 0 and 2 into rows 1 and 3) and
// row_bcast:31 (lane 31 into rows 2 and 3).  The whole wave must be active.
// (A shuffle per step goes through the LDS crossbar, one round trip each;
// these stay in the vector ALU.)  Lanes a move leaves without a source
// take the operation's identity.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}
__device__ __forceinline__ uint32_t wave_incl_min(uint32_t x) {
  constexpr uint32_t I = 0xFFFFFFFFu;
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(I, x, 0x111, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(I, x, 0x112, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(I, x, 0x114, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(I, x, 0x118, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(I, x, 0x142, 0xA, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(I, x, 0x143, 0xC, 0xF, false));
  return x;
}
__device__ __forceinline__ uint32_t wave_incl_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false));
  return x;
}

// Exclusive prefix sum over the workgroup in thread order.  tmp needs
// NT/64 + 1 words of LDS.  Returns this thread's exclusive prefix; *total
// receives the sum over all threads.
template <int NT>
__device__ __forceinline__ uint32_t block_exscan(uint32_t v, uint32_t* tmp,
                                                 uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t x = wave_incl_sum(v);
  if (lane == 63) tmp[wv] = x;
  __syncthreads();
  if (wv == 0) {
    const uint32_t t = lane < NW ? tmp[lane] : 0u;
    const uint32_t ti = wave_incl_sum(t);
    if (lane < NW) tmp[lane] = ti - t;
    if (lane == NW - 1) tmp[NW] = ti;
  }
  __syncthreads();
  const uint32_t res = tmp[wv] + x - v;
  *total = tmp[NW];
  __syncthreads();
  return res;
}

// The same over uint64 values; used with several 16-bit counts packed in
// one word (each field's total must stay below 2^16, so the low 32 bits
// never carry into the high 32 and each half is scanned on its own).
// tmp: NT/64 + 1 words.
template <int NT>
__device__ __forceinline__ uint64_t block_exscan_u64(uint64_t v, uint64_t* tmp,
                                                     uint64_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t x = ((uint64_t)wave_incl_sum((uint32_t)(v >> 32)) << 32) |
                     wave_incl_sum((uint32_t)v);
  if (lane == 63) tmp[wv] = x;
  __syncthreads();
  if (wv == 0) {
    const uint64_t t = lane < NW ? tmp[lane] : 0ull;
    const uint64_t ti = ((uint64_t)wave_incl_sum((uint32_t)(t >> 32)) << 32) |
                        wave_incl_sum((uint32_t)t);
    if (lane < NW) tmp[lane] = ti - t;
    if (lane == NW - 1) tmp[NW] = ti;
  }
  __syncthreads();
  const uint64_t res = tmp[wv] + x - v;
  *total = tmp[NW];
  __syncthreads();
  return res;
}

// Minimum and maximum of a uint32 over the workgroup.  tmp: 2*(NT/64) words.
template <int NT>
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx,
                                             uint32_t* tmp) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  mn = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_min(mn), 63);
  mx = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_max(mx), 63);
  if (lane == 0) {
    tmp[wv] = mn;
    tmp[NW + wv] = mx;
  }
  __syncthreads();
  mn = tmp[0];
  mx = tmp[NW];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    mn = min(mn, tmp[i]);
    mx = max(mx, tmp[NW + i]);
  }
  __syncthreads();
}

// In-place bitonic sort of n (a power of two) 64-bit keys in LDS.
// DESC: largest first.  Ends with a barrier.
template <int NT, bool DESC>
__device__ void bitonic_sort_u64(uint64_t* a, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int q = threadIdx.x; q < (n >> 1); q += NT) {
        const int i = ((q & ~(stride - 1)) << 1) | (q & (stride - 1));
        const int j = i + stride;
        const bool up = ((i & size) == 0) == DESC;  // block wants larger first
        const uint64_t x = a[i], y = a[j];
        if (up ? (x < y) : (x > y)) {
          a[i] = y;
          a[j] = x;
        }
      }
      __syncthreads();
    }
  }
}

// Bitonic sort of n = NT * E 64-bit keys (n a power of two) held in LDS,
// done mostly in registers: thread t keeps elements r * NT + t (r < E).
// Compare-exchange partners at stride < 64 are in the same wave (lane
// shuffles), at stride >= NT in the same thread, and only strides 64..NT/2
// go through LDS.  DESC: largest first.  Ends with the sorted keys back in
// `a` and a barrier.
template <int NT, bool DESC, int E>
__device__ __forceinline__ void block_sort_u64(uint64_t* a) {
  constexpr int n = NT * E;
  const int t = threadIdx.x;
  uint64_t v[E];
#pragma unroll
  for (int r = 0; r < E; ++r) v[r] = a[r * NT + t];
  // Keep the larger of a pair at its lower index in blocks that sort
  // downward (DESC: the blocks with bit `size` clear).
  auto want_max = [](int i, int p, int size) {
    const bool lower = i < p;
    const bool down = ((i & size) == 0) == DESC;
    return lower == down;
  };
#pragma unroll 1
  for (int size = 2; size <= n; size <<= 1) {
#pragma unroll 1
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= NT) {
        // Partners in the same thread: register index r ^ rs.  rs takes
        // each power of two below E as a compile-time constant, so v stays
        // in registers (a runtime index would put it in scratch memory).
#pragma unroll
        for (int rs = 1; rs < E; rs <<= 1) {
          if (stride != rs * NT) continue;
#pragma unroll
          for (int r = 0; r < E; ++r) {
            if (r & rs) continue;
            const int i = r * NT + t;
            const uint64_t x = v[r], y = v[r ^ rs];
            const bool wm = want_max(i, i ^ stride, size);
            v[r] = wm ? (x > y ? x : y) : (x < y ? x : y);
            v[r ^ rs] = wm ? (x > y ? y : x) : (x < y ? y : x);
          }
        }
      } else if (stride >= 64) {
#pragma unroll
        for (int r = 0; r < E; ++r) a[r * NT + t] = v[r];
        __syncthreads();
#pragma unroll
        for (int r = 0; r < E; ++r) {
          const int i = r * NT + t;
          const uint64_t y = a[i ^ stride];
          const uint64_t x = v[r];
          v[r] = want_max(i, i ^ stride, size) ? (x > y ? x : y) : (x < y ? x : y);
        }
        __syncthreads();
      } else {
#pragma unroll
        for (int r = 0; r < E; ++r) {
          const int i = r * NT + t;
          const uint32_t lo = (uint32_t)v[r], hi = (uint32_t)(v[r] >> 32);
          const uint64_t y = ((uint64_t)(uint32_t)__shfl_xor((int)hi, stride) << 32) |
                             (uint32_t)__shfl_xor((int)lo, stride);
          const uint64_t x = v[r];
          v[r] = want_max(i, i ^ stride, size) ? (x > y ? x : y) : (x < y ? x : y);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < E; ++r) a[r * NT + t] = v[r];
  __syncthreads();
}

// block_sort_u64 for any power-of-two n in [NT, 16 NT].
template <int NT, bool DESC>
__device__ __forceinline__ void block_sort_u64_n(uint64_t* a, int n) {
  switch (n / NT) {
    case 1: block_sort_u64<NT, DESC, 1>(a); break;
    case 2: block_sort_u64<NT, DESC, 2>(a); break;
    case 4: block_sort_u64<NT, DESC, 4>(a); break;
    case 8: block_sort_u64<NT, DESC, 8>(a); break;
    default: block_sort_u64<NT, DESC, 16>(a); break;
  }
}

// Bucket sort of n 64-bit keys in LDS: histogram over nb buckets (a
// multiple of NT), exclusive scan, scatter into the scratch array g grouped
// by bucket, then every key finds its place by counting the keys of its own
// bucket that go before it (equal keys keep their grouped order), so the
// cost grows with the largest bucket rather than its square, and no thread
// walks a bucket alone.  The sorted keys end back in a.  bucket(key) must be
// monotone in the output order (DESC: larger keys never in a later bucket).
// Returns false - with a unchanged - when a bucket holds more than
// max_bucket keys; the caller then sorts another way.  cnt: nb words of LDS;
// tmp: NT/64 + 1 words.  Ends with a barrier.
template <int NT, bool DESC, typename BucketFn>
__device__ bool bucket_sort_u64(uint64_t* a, uint64_t* g, int n, int nb,
                                BucketFn bucket, uint32_t* cnt, uint32_t* tmp,
                                int max_bucket) {
  const int t = threadIdx.x;
  const int bpt = nb / NT;   // buckets per thread
  for (int i = t; i < nb; i += NT) cnt[i] = 0;
  __syncthreads();
  for (int i = t; i < n; i += NT) atomicAdd(&cnt[bucket(a[i])], 1u);
  __syncthreads();
  uint32_t mine = 0, big = 0;
  for (int q = 0; q < bpt; ++q) {
    const uint32_t c = cnt[t * bpt + q];
    mine += c;
    big = max(big, c);
  }
  uint32_t tot;
  uint32_t off = block_exscan<NT>(mine, tmp, &tot);
  const bool too_big = __syncthreads_or(big > (uint32_t)max_bucket);
  if (too_big) return false;
  for (int q = 0; q < bpt; ++q) {
    const uint32_t c = cnt[t * bpt + q];
    cnt[t * bpt + q] = off;      // fill cursor = bucket start
    off += c;
  }
  __syncthreads();
  for (int i = t; i < n; i += NT) {
    const uint64_t x = a[i];
    g[atomicAdd(&cnt[bucket(x)], 1u)] = x;
  }
  __syncthreads();
  // cnt[b] is now the end of bucket b, so bucket b spans [cnt[b-1], cnt[b]).
  for (int i = t; i < n; i += NT) {
    const uint64_t x = g[i];
    const int b = bucket(x);
    const int lo = b == 0 ? 0 : (int)cnt[b - 1], hi = (int)cnt[b];
    int r = lo;
    for (int q = lo; q < hi; ++q) {
      const uint64_t y = g[q];
      r += (DESC ? y > x : y < x) || (y == x && q < i);
    }
    a[r] = x;
  }
  __syncthreads();
  return true;
}

// Bitonic sort across the 64 lanes of one wave, one key per lane (lane i
// ends with the i-th key in order).  Must be reached by the whole wave.
template <bool DESC>
__device__ __forceinline__ uint64_t wave_bitonic_u64(uint64_t x, int i) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
      const uint64_t y = ((uint64_t)(uint32_t)__shfl_xor((int)hi, stride) << 32) |
                         (uint32_t)__shfl_xor((int)lo, stride);
      const bool lower = (i & stride) == 0;
      const bool down = ((i & size) == 0) == DESC;
      x = (lower == down) ? (x > y ? x : y) : (x < y ? x : y);
    }
  }
  return x;
}

// Bitonic sort of up to 64 keys by one wave (wave 0), one key per lane;
// lanes past n hold `pad`, which must sort after every real key.  Other
// waves just wait at the closing barrier.
template <bool DESC>
__device__ void wave_sort_u64(uint64_t* a, int n, uint64_t pad) {
  if (threadIdx.x < 64) {
    const int i = threadIdx.x;
    const uint64_t x = wave_bitonic_u64<DESC>(i < n ? a[i] : pad, i);
    if (i < n) a[i] = x;
  }
  __syncthreads();
}

}  // namespace ess
