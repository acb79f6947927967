// Copy of a miss list from mapped pinned host memory into pool slots: the
// H2D load of the copy triples (FlashOffloading analysis, section "five
// steps and the MTP union", step 5) and the ESS small-block transfer of
// latent entries (ESS concept page, "core mechanism" table).  Done inside a
// kernel with 16-byte loads through the device view of the host buffer, so
// many scattered 1152-byte rows are in flight at once instead of one DMA
// descriptor per row.
#include "ess_internal.h"
#include "fp8_entry.h"

namespace ess {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
constexpr int NT = 256;
constexpr int kPieces = kLat / 8;   // 16-byte pieces per row
constexpr int kChunksPerRow = kPieces;
constexpr int kInFlight = 8;        // 16-byte host reads in flight per thread
constexpr int kTargetWgs = 128;     // whole grid, all requests

// A small grid whose threads each keep kInFlight host reads in flight: the
// host link needs only a few hundred KB outstanding to run at its rate, and
// a small grid leaves most CUs free for work running beside the copy (a
// grid of one read per thread would hold every CU's wave slots while its
// reads wait on the link).
__global__ __launch_bounds__(NT) void miss_copy_kernel(
    int list_stride, const int32_t* __restrict__ miss_pos,
    const int32_t* __restrict__ miss_slot, const int32_t* __restrict__ n_miss,
    const uint16_t* __restrict__ host, uint16_t* __restrict__ pool, int L,
    int C) {
  const int b = blockIdx.y;
  const int nm = n_miss[b];
  const int32_t* mp = miss_pos + (size_t)b * list_stride;
  const int32_t* ms = miss_slot + (size_t)b * list_stride;
  const uint16_t* hb = host + (size_t)b * L * kLat;
  uint16_t* pb = pool + (size_t)b * C * kLat;
  const int total = min(nm, list_stride) * kPieces;
  const int stride = gridDim.x * NT;
  for (int i0 = blockIdx.x * NT + threadIdx.x; i0 < total; i0 += stride * kInFlight) {
    v4u buf[kInFlight];
    int dst[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int idx = i0 + u * stride;
      dst[u] = -1;
      if (idx < total) {
        const int q = idx / kPieces, ch = idx - q * kPieces;
        const int pos = mp[q], slot = ms[q];
        if (pos >= 0 && pos < L && slot >= 0 && slot < C) {
          buf[u] = *reinterpret_cast<const v4u*>(hb + (size_t)pos * kLat + ch * 8);
          dst[u] = slot * kChunksPerRow + ch;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      if (dst[u] >= 0)
        *reinterpret_cast<v4u*>(pb + (size_t)dst[u] * 8) = buf[u];
  }
}

// ---- 656-byte fp8 entries ------------------------------------------------
// The copy reads each entry once from host memory into LDS and writes the
// pool row as bf16 (c_KV dequantized with its block's scale, k_R as stored).
constexpr int kEntriesPerIter = 48;                       // per workgroup pass
constexpr int kEntryLoads = (kEntriesPerIter * kEntryPieces + NT - 1) / NT;   // 8

__global__ __launch_bounds__(NT) void entry_copy_kernel(
    int list_stride, const int32_t* __restrict__ miss_pos,
    const int32_t* __restrict__ miss_slot, const int32_t* __restrict__ n_miss,
    const unsigned char* __restrict__ host, uint16_t* __restrict__ pool, int L,
    int C) {
  __shared__ v4u stage[kEntriesPerIter * kEntryPieces];
  __shared__ int dst_slot[kEntriesPerIter];
  const int b = blockIdx.y;
  const int nm = min(n_miss[b], list_stride);
  const int32_t* mp = miss_pos + (size_t)b * list_stride;
  const int32_t* ms = miss_slot + (size_t)b * list_stride;
  const unsigned char* hb = host + (size_t)b * L * kEntryBytes;
  uint16_t* pb = pool + (size_t)b * C * kLat;
  // The pass loop is uniform over the workgroup (it depends on blockIdx and
  // nm only), so the barriers inside it are reached by every thread.
  for (int q0 = blockIdx.x * kEntriesPerIter; q0 < nm;
       q0 += gridDim.x * kEntriesPerIter) {
    v4u buf[kEntryLoads];
    bool got[kEntryLoads];
#pragma unroll
    for (int u = 0; u < kEntryLoads; ++u) {
      const int idx = threadIdx.x + u * NT;
      const int e = idx / kEntryPieces, piece = idx - e * kEntryPieces;
      got[u] = false;
      if (e < kEntriesPerIter && q0 + e < nm) {
        const int pos = mp[q0 + e];
        if (pos >= 0 && pos < L) {
          buf[u] = *reinterpret_cast<const v4u*>(hb + (size_t)pos * kEntryBytes + piece * 16);
          got[u] = true;
        }
      }
    }
    if (threadIdx.x < kEntriesPerIter) {
      const int q = q0 + threadIdx.x;
      int slot = -1;
      if (q < nm) {
        const int pos = mp[q], s = ms[q];
        if (pos >= 0 && pos < L && s >= 0 && s < C) slot = s;
      }
      dst_slot[threadIdx.x] = slot;
    }
#pragma unroll
    for (int u = 0; u < kEntryLoads; ++u)
      if (got[u]) stage[threadIdx.x + u * NT] = buf[u];
    __syncthreads();
    for (int o = threadIdx.x; o < kEntriesPerIter * kPieces; o += NT) {
      const int e = o / kPieces, p = o - e * kPieces;
      const int slot = dst_slot[e];
      if (slot < 0) continue;
      const unsigned char* ent = reinterpret_cast<const unsigned char*>(stage + e * kEntryPieces);
      v4u w;
      if (p < kVal / 8) {
        const uint2 q8 = *reinterpret_cast<const uint2*>(ent + p * 8);
        const float sc = *reinterpret_cast<const float*>(ent + kEntryScaleOff + (p / 16) * 4);
        w = dequant8(q8.x, q8.y, sc);
      } else {
        w = *reinterpret_cast<const v4u*>(ent + kEntryRopeOff + (p - kVal / 8) * 16);
      }
      *reinterpret_cast<v4u*>(pb + ((size_t)slot * kPieces + p) * 8) = w;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_miss_copy(const ess_dims& d, int list_stride,
                            const int32_t* miss_pos, const int32_t* miss_slot,
                            const int32_t* n_miss, const uint16_t* host,
                            uint16_t* pool, hipStream_t s) {
  // About kTargetWgs workgroups over all requests; the loop strides over
  // whatever the miss count turns out to be.
  int gx = (kTargetWgs + d.batch - 1) / d.batch;
  const int need = (list_stride * kPieces + NT * kInFlight - 1) / (NT * kInFlight);
  if (gx > need) gx = need;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL(miss_copy_kernel, dim3(gx, d.batch), dim3(NT), 0, s,
                     list_stride, miss_pos, miss_slot, n_miss, host, pool,
                     d.ctx_len, d.pool_slots);
  return hipGetLastError();
}

hipError_t launch_entry_copy(const ess_dims& d, int list_stride,
                             const int32_t* miss_pos, const int32_t* miss_slot,
                             const int32_t* n_miss, const uint8_t* host,
                             uint16_t* pool, hipStream_t s) {
  int gx = (kTargetWgs + d.batch - 1) / d.batch;
  const int need = (list_stride + kEntriesPerIter - 1) / kEntriesPerIter;
  if (gx > need) gx = need;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL(entry_copy_kernel, dim3(gx, d.batch), dim3(NT), 0, s,
                     list_stride, miss_pos, miss_slot, n_miss, host, pool,
                     d.ctx_len, d.pool_slots);
  return hipGetLastError();
}

}  // namespace ess
