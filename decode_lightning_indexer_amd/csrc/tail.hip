// Growing context: each decode step appends its new tokens' index keys to
// the resident index cache and their latents to the request's open tail
// block in device memory (FlashOffloading analysis, architecture section and
// Fig. 2: beside the hot cache, decode keeps two tail blocks that take the
// new KV).  The block bookkeeping and the write-back to the host store are
// in the C-ABI layer.
#include "ess_internal.h"
#include "fp8_entry.h"

namespace ess {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
constexpr int NT = 256;
constexpr int kPieces = kLat / 8;   // 16-byte pieces per latent row

// One workgroup per request: keys of the m new tokens to k_idx[b][n_ctx + j],
// latents to their tail rows, the visible lengths n_vis[b][j] = n_ctx + 1 + j
// (token j sees every position up to its own), then the request's length and
// first tail position advance.  state = (first[B], n_ctx[B], start[B]).
__global__ __launch_bounds__(NT) void append_tokens_kernel(
    int m, int L, int idx_dim, int block, const unsigned char* __restrict__ new_keys,
    const uint16_t* __restrict__ new_lat, unsigned char* __restrict__ k_idx,
    uint16_t* __restrict__ tail, unsigned char* __restrict__ tail_ent,
    int32_t* __restrict__ n_vis, int32_t* __restrict__ state) {
  const int b = blockIdx.x, B = gridDim.x;
  const int first = state[b], n_ctx = state[B + b];
  const int key_bytes = m * idx_dim;
  const unsigned char* ks = new_keys + (size_t)b * key_bytes;
  unsigned char* kd = k_idx + ((size_t)b * L + n_ctx) * idx_dim;
  for (int i = threadIdx.x; i < key_bytes / 16; i += NT)
    reinterpret_cast<v4u*>(kd)[i] = reinterpret_cast<const v4u*>(ks)[i];
  if (tail_ent == nullptr) {
    for (int i = threadIdx.x; i < m * kPieces; i += NT) {
      const int j = i / kPieces, pc = i - j * kPieces;
      const int pos = n_ctx + j;
      const int row = ((pos / block) & 1) * block + pos % block;
      const v4u v = reinterpret_cast<const v4u*>(new_lat + ((size_t)b * m + j) * kLat)[pc];
      reinterpret_cast<v4u*>(tail + ((size_t)b * 2 * block + row) * kLat)[pc] = v;
    }
  } else {
    // Entry store: each new latent is quantized into its 656-byte entry and
    // the tail row holds the entry dequantized, so a position reads the
    // same values from the tail, the pool or (after write-back) the host
    // store.  Threads 0-127 take four c_KV values each (32 threads per
    // 128-value block), threads 128-191 one k_R value each.
    const int t = threadIdx.x;
    for (int j = 0; j < m; ++j) {
      const int pos = n_ctx + j;
      const int row = ((pos / block) & 1) * block + pos % block;
      const uint16_t* src = new_lat + ((size_t)b * m + j) * kLat;
      uint16_t* dst = tail + ((size_t)b * 2 * block + row) * kLat;
      unsigned char* ent = tail_ent + ((size_t)b * 2 * block + row) * kEntryBytes;
      if (t < kVal / 4) {
        const uint2 w = reinterpret_cast<const uint2*>(src)[t];
        const float x[4] = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                            __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
        float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        const int te = entry_scale_exp(amax);
        unsigned q = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) q |= f32_to_e4m3fn_rne(ldexpf(x[e], -te)) << (8 * e);
        reinterpret_cast<unsigned*>(ent)[t] = q;
        const float sc = ldexpf(1.f, te);
        if ((t & 31) == 0) reinterpret_cast<float*>(ent + kEntryScaleOff)[t >> 5] = sc;
        const entry_v4u d = dequant8(q, 0u, sc);
        reinterpret_cast<uint2*>(dst)[t] = make_uint2(d.x, d.y);
      } else if (t < kVal / 4 + (kLat - kVal)) {
        const int r = t - kVal / 4;
        reinterpret_cast<uint16_t*>(ent + kEntryRopeOff)[r] = src[kVal + r];
        dst[kVal + r] = src[kVal + r];
      }
    }
  }
  if (threadIdx.x < m) n_vis[b * m + threadIdx.x] = n_ctx + 1 + threadIdx.x;
  __syncthreads();                      // every thread has read n_ctx (and,
                                        // with entries, the rows are written)
  if (threadIdx.x == 0) {
    const int n1 = n_ctx + m;
    state[B + b] = n1;
    state[2 * B + b] = max(first, ((n1 - 1) / block - 1) * block);
  }
}

}  // namespace

hipError_t launch_append_tokens(const ess_dims& d, int block,
                                const uint8_t* new_keys,
                                const uint16_t* new_lat, uint8_t* k_idx,
                                uint16_t* tail, uint8_t* tail_ent,
                                int32_t* n_vis, int32_t* state, hipStream_t s) {
  hipLaunchKernelGGL(append_tokens_kernel, dim3(d.batch), dim3(NT), 0, s,
                     d.mtp, d.ctx_len, d.idx_dim, block, new_keys, new_lat,
                     k_idx, tail, tail_ent, n_vis, state);
  return hipGetLastError();
}

}  // namespace ess
