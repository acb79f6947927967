// Kernels of the four-buffer prefill pipeline: the stand-in layer compute
// (append the chunk's new rows after the layer's history in its buffer, then
// reduce every row of the buffer to per-column sums) whose result shows it
// consumed exactly the loaded history plus the new rows.  The pipeline that
// binds buffers, loads, computes and writes back is in the C-ABI layer
// (FlashOffloading analysis, prefill section: four full-layer buffers, a
// five-step layer lifecycle, Figs. 2 and 3).
#include <algorithm>

#include "ess_internal.h"

namespace ess {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kPieces = kLat / 8;          // 16-byte pieces per row (72)
constexpr int kRowLanes = 8;               // row lanes per workgroup
constexpr int kSumThreads = kPieces * kRowLanes;   // 576
constexpr int kRowsPerBlock = 128;         // rows a workgroup holds in registers
constexpr int kRowsPerLane = kRowsPerBlock / kRowLanes;   // 16
constexpr int kRedCols = 64, kRedLanes = 16;               // reduce: 1024 threads

// Copy n rows of 576 bf16 from src to dst (both device), 16 bytes a thread.
__global__ __launch_bounds__(256) void append_rows_kernel(
    const v4u* __restrict__ src, v4u* __restrict__ dst, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

// Per-column sums of rows [blk * kRowsPerBlock, ...) of a [rows][576] bf16
// buffer into part[blk][576].  The workgroup reads its rows from memory
// once - thread (lane r, piece p) keeps piece p of rows r, r + 8, ... in
// registers - and then sums them `reps` times on chip: the repetitions set
// the length of the layer's compute the way a layer's attention and FFN
// would, reading the layer's KV once and then working on chip (re-reading
// the buffer per repetition would make the stand-in's time depend on the
// last-level cache the concurrent loads also fill).  Every repetition gives
// the same sums: the thread adds the 8 columns of its piece over its rows,
// then the 8 row lanes are added in LDS in fixed order.
__global__ __launch_bounds__(kSumThreads) void column_sums_kernel(
    const v4u* __restrict__ buf, int rows, int reps, float* __restrict__ part) {
  __shared__ float acc[kRowLanes][kLat];
  const int p = threadIdx.x % kPieces, r = threadIdx.x / kPieces;
  const int r0 = blockIdx.x * kRowsPerBlock;
  v4u v[kRowsPerLane];
#pragma unroll
  for (int i = 0; i < kRowsPerLane; ++i) {
    const int row = r0 + r + i * kRowLanes;
    v[i] = row < rows ? buf[(size_t)row * kPieces + p] : v4u{0u, 0u, 0u, 0u};
  }
  const int c = threadIdx.x;             // one column per thread in the fold
  float t = 0.f;
  for (int rep = 0; rep < reps; ++rep) {
    // (the rows are taken as unknown again, so each repetition sums them)
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) asm volatile("" : "+v"(v[i]));
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
      s[0] += bf16_lo(v[i].x); s[1] += bf16_hi(v[i].x);
      s[2] += bf16_lo(v[i].y); s[3] += bf16_hi(v[i].y);
      s[4] += bf16_lo(v[i].z); s[5] += bf16_hi(v[i].z);
      s[6] += bf16_lo(v[i].w); s[7] += bf16_hi(v[i].w);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][p * 8 + e] = s[e];
    __syncthreads();
    t = 0.f;
#pragma unroll
    for (int q = 0; q < kRowLanes; ++q) t += acc[q][c];
    __syncthreads();                     // acc read before it is written again
  }
  part[(size_t)blockIdx.x * kLat + c] = t;
}

// out[c] = sum over blocks of part[blk][c]: 16 lanes per column each add
// every 16th block (their loads in flight together), then the lanes are
// added in fixed order.
__global__ __launch_bounds__(kRedCols * kRedLanes) void column_sums_reduce_kernel(
    const float* __restrict__ part, int nblk, float* __restrict__ out) {
  __shared__ float acc[kRedLanes][kRedCols];
  const int cl = threadIdx.x % kRedCols, q = threadIdx.x / kRedCols;
  const int c = blockIdx.x * kRedCols + cl;
  float t = 0.f;
#pragma unroll 4
  for (int b = q; b < nblk; b += kRedLanes) t += part[(size_t)b * kLat + c];
  acc[q][cl] = t;
  __syncthreads();
  if (q == 0) {
    float u = 0.f;
#pragma unroll
    for (int i = 0; i < kRedLanes; ++i) u += acc[i][cl];
    out[c] = u;
  }
}

static_assert(kLat % kRedCols == 0, "reduce covers the columns in whole workgroups");

}  // namespace

size_t prefill_ws_bytes(int rows) {
  const size_t nblk = ((size_t)rows + kRowsPerBlock - 1) / kRowsPerBlock;
  return nblk * kLat * sizeof(float);
}

hipError_t launch_prefill_compute(const uint16_t* new_rows, int n_new,
                                  uint16_t* buf, int n_hist, int reps,
                                  float* part, float* out, hipStream_t s) {
  if (n_new > 0) {
    const size_t n16 = (size_t)n_new * kPieces;
    const unsigned grid = (unsigned)std::min<size_t>((n16 + 255) / 256, 1024);
    hipLaunchKernelGGL(append_rows_kernel, dim3(grid), dim3(256), 0, s,
                       reinterpret_cast<const v4u*>(new_rows),
                       reinterpret_cast<v4u*>(buf + (size_t)n_hist * kLat), n16);
  }
  const int rows = n_hist + n_new;
  const int nblk = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(column_sums_kernel, dim3(nblk), dim3(kSumThreads), 0, s,
                     reinterpret_cast<const v4u*>(buf), rows, reps, part);
  hipLaunchKernelGGL(column_sums_reduce_kernel, dim3(kLat / kRedCols),
                     dim3(kRedCols * kRedLanes), 0, s, part, nblk, out);
  return hipGetLastError();
}

}  // namespace ess
