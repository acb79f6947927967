// Copy of a miss list from mapped pinned host memory into pool slots: the
// H2D load of the copy triples (FlashOffloading analysis, section "five
// steps and the MTP union", step 5) and the ESS small-block transfer of
// latent entries (ESS concept page, "core mechanism" table).  Done inside a
// kernel with 16-byte loads through the device view of the host buffer, so
// many scattered 1152-byte rows are in flight at once instead of one DMA
// descriptor per row.
#include "ess_internal.h"

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

}  // namespace ess
