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

// Exclusive prefix sum over the workgroup in thread order.  tmp needs
// NT/64 + 1 words of LDS.  Returns this thread's exclusive prefix; *total
// receives the sum over all threads.
template <int NT>
__device__ __forceinline__ uint32_t block_exscan(uint32_t v, uint32_t* tmp,
                                                 uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wv] = x;
  __syncthreads();
  if (wv == 0) {
    uint32_t t = lane < NW ? tmp[lane] : 0u;
    uint32_t ti = t;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
      uint32_t y = __shfl_up(ti, o);
      if (lane >= o) ti += y;
    }
    if (lane < NW) tmp[lane] = ti - t;
    if (lane == NW - 1) tmp[NW] = ti;
  }
  __syncthreads();
  const uint32_t res = tmp[wv] + x - v;
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
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor(mn, o));
    mx = max(mx, (uint32_t)__shfl_xor(mx, o));
  }
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

}  // namespace ess
