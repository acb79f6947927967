// Growing context: each decode step appends its new tokens' index keys to
// the resident index cache and their latents to the request's open tail
// block in device memory (FlashOffloading analysis, architecture section and
// Fig. 2: beside the hot cache, decode keeps two tail blocks that take the
// new KV).  The block bookkeeping and the write-back to the host store are
// in the C-ABI layer.
#include "ess_internal.h"

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
    uint16_t* __restrict__ tail, int32_t* __restrict__ n_vis,
    int32_t* __restrict__ state) {
  const int b = blockIdx.x, B = gridDim.x;
  const int first = state[b], n_ctx = state[B + b];
  const int key_bytes = m * idx_dim;
  const unsigned char* ks = new_keys + (size_t)b * key_bytes;
  unsigned char* kd = k_idx + ((size_t)b * L + n_ctx) * idx_dim;
  for (int i = threadIdx.x; i < key_bytes / 16; i += NT)
    reinterpret_cast<v4u*>(kd)[i] = reinterpret_cast<const v4u*>(ks)[i];
  for (int i = threadIdx.x; i < m * kPieces; i += NT) {
    const int j = i / kPieces, pc = i - j * kPieces;
    const int pos = n_ctx + j;
    const int row = ((pos / block) & 1) * block + pos % block;
    const v4u v = reinterpret_cast<const v4u*>(new_lat + ((size_t)b * m + j) * kLat)[pc];
    reinterpret_cast<v4u*>(tail + ((size_t)b * 2 * block + row) * kLat)[pc] = v;
  }
  if (threadIdx.x < m) n_vis[b * m + threadIdx.x] = n_ctx + 1 + threadIdx.x;
  __syncthreads();                      // every thread has read n_ctx
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
                                uint16_t* tail, int32_t* n_vis,
                                int32_t* state, hipStream_t s) {
  hipLaunchKernelGGL(append_tokens_kernel, dim3(d.batch), dim3(NT), 0, s,
                     d.mtp, d.ctx_len, d.idx_dim, block, new_keys, new_lat,
                     k_idx, tail, n_vis, state);
  return hipGetLastError();
}

}  // namespace ess
