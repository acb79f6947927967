// Lightning-indexer scores over every cached position, fp8 MFMA on gfx950.
//
// The indexer cache is the part of the DSA cache that stays in device memory
// and is scanned in full every step (ESS concept page, "dual cache" table);
// it is what grows with context in device memory (FlashOffloading analysis,
// section "how 95.23 kB per token comes about").  The scan is therefore
// bandwidth-bound: 2 * m * H_I flops per key byte is far below the fp8
// MFMA ridge.  MFMA keeps the arithmetic off the critical path.
//
// Mapping onto v_mfma_f32_16x16x128_f8f6f4 (A: 16x128, B: 128x16, D: 16x16):
//   A = 16 query heads x 128 dims (held in registers for the whole kernel),
//   B = 128 dims x 16 positions (32 bytes of a key row per lane, two
//       16-byte loads),
//   D[head][pos] -> each lane holds 4 heads of one position; it applies the
//   ReLU and head weight to its 4 heads, and two lane exchanges finish the
//   head sum.  Lane group g (lanes 16g..16g+15) feeds the same 32 dims of
//   both operands, so A and B agree on the reduction index.
// Inputs with integer values in [-7, 7] and integer weights keep every
// partial sum an integer below 2^24, so the fp32 result is exact.
#include "ess_internal.h"

namespace ess {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;     // 4 waves
constexpr int kGroups = 4;        // 16-position groups per wave iteration
constexpr int kSpan = 1024;       // positions per workgroup

// The 32 reduction-index bytes of a row held by lane group g: bytes
// [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16) (zeros past a 64-wide
// row).  Queries and keys use the same assignment, so the reduction is
// unchanged, and each of the two loads of a wave reads 64 contiguous bytes
// of each of its 16 rows.  Key rows are streamed once per step, so they are
// loaded non-temporally.
template <int DI, bool STREAM>
__device__ __forceinline__ v8i load_piece(const uint8_t* row, int g) {
  const v4u* p = reinterpret_cast<const v4u*>(row + g * 16);
  v4u a, b = {0u, 0u, 0u, 0u};
  if (STREAM) {
    a = __builtin_nontemporal_load(p);
    if (DI == 128) b = __builtin_nontemporal_load(p + 4);
  } else {
    a = p[0];
    if (DI == 128) b = p[4];
  }
  v8i v = {(int)a.x, (int)a.y, (int)a.z, (int)a.w,
           (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  return v;
}

// Key rows are staged through LDS so that the loads from memory are fully
// contiguous: each wave owns two buffers of 64 rows and copies its next 64
// rows (DI * 64 contiguous bytes) with gfx950's 16-byte global-to-LDS load,
// one 1 KB block per wave instruction, while it computes the current 64.
// Rows are stored unpadded, with the 16-byte pieces of each row permuted
// (piece p of buffer row r at slot p ^ f(r), f(r) = (r / (256 / DI)) mod
// (DI / 16)): the 16 rows that the 16 lanes of a lane group read for one
// operand then fall in 16 different 16-byte bank groups, so the operand
// reads are conflict-free, and every load still reads one contiguous 1 KB
// block (the permutation stays within rows).  A wave reads only its own
// buffers, so its own vmcnt wait is all the synchronisation needed.
constexpr int kRows = kGroups * 16;   // rows per wave iteration

// One wave instruction: lane l copies the 16 bytes at base + off to LDS at
// lds_block + 16 l.  base is the same for the whole wave (scalar registers),
// off a 32-bit per-lane byte offset.
__device__ __forceinline__ void load_lds16(const uint8_t* base, uint32_t off,
                                           const void* lds_block) {
  const unsigned lds = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(
      const __attribute__((address_space(3))) void*)lds_block);
  // readfirstlane returns int: each half goes through uint32_t so that the
  // low half is zero-extended (a sign-extended low half with bit 31 set would
  // fill the upper half with ones).
  const uint64_t b64 = (uint64_t)(uintptr_t)base;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(b64 >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)b64);
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  // An SALU write of M0 needs one wait state before an LDS-DMA load reads it.
  // The key rows are read once per step: the non-temporal hint keeps them
  // from displacing other lines (measured from HBM at 32K x 16: 15.1 ->
  // 13.8 us per launch).
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :: "s"(lds), "v"(off), "s"(sb) : "memory", "m0");
}

template <int DI>
struct Stage {
  static constexpr int kSlots = DI / 16;               // 16-byte pieces per row
  static constexpr int kPerBank = 256 / DI;            // rows per 256 bytes
  static constexpr int kLoads = kRows * kSlots / 64;   // wave loads per 64 rows
  static constexpr int kBytes = kRows * DI;            // one buffer
  // Slot of piece p of buffer row r.
  static __device__ __forceinline__ int slot(int r, int p) {
    return p ^ ((r / kPerBank) % kSlots);
  }
};

// NT: 16-row tiles of the [m * H_I][DI] query matrix; MT: query tokens m.
template <int DI, int NT, int MT>
__global__ __launch_bounds__(kThreads) void index_scores_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ w,
    const uint8_t* __restrict__ keys, const int32_t* __restrict__ n_vis,
    float* __restrict__ scores, int L, int HI, ClearSpec clr) {
  using S = Stage<DI>;
  if (clr.base) {
    // Zero the following selection's control words, spread over the grid.
    const size_t total = (size_t)clr.rows * clr.words;
    const size_t step = (size_t)gridDim.x * gridDim.y * kThreads;
    for (size_t i = ((size_t)blockIdx.y * gridDim.x + blockIdx.x) * kThreads + threadIdx.x;
         i < total; i += step)
      clr.base[(i / clr.words) * clr.stride_words + i % clr.words] = 0u;
  }
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;   // lane group: reduction slice / output rows
  const int c = lane & 15;   // position within a 16-group / head row
  const int b = blockIdx.y;
  uint8_t* buf0 = smem + (size_t)wave * 2 * S::kBytes;

  // Query tiles and head weights for this lane, resident in registers.
  constexpr int kTilesPerTok = NT / MT;   // a 16-row tile never straddles tokens
  v8i qa[NT];
  float wv[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int row = t * 16 + c;                      // flattened (j, h)
    qa[t] = load_piece<DI, false>(q + ((size_t)b * MT * HI + row) * DI, g);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      wv[t][r] = w[(size_t)b * MT * HI + t * 16 + g * 4 + r];
  }
  int nv[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) nv[j] = n_vis[b * MT + j];

  const int span0 = blockIdx.x * kSpan;
  const int span1 = min(L, span0 + kSpan);
  // The staging loads take a 64-bit base at this workgroup's first row and
  // a 32-bit lane offset below kSpan * DI bytes, so no offset wraps however
  // long the context is.
  const uint8_t* kb = keys + ((size_t)b * L + span0) * DI;

  // Copy rows [p, p + kRows) into buffer `which`: load j writes slots
  // 64 j .. 64 j + 63, i.e. rows 64 j / kSlots + lane / kSlots, slot
  // lane % kSlots, which holds piece slot ^ f(row) of the row (rows past L
  // repeat row L - 1).
  const int lr = lane / S::kSlots, ls = lane % S::kSlots;
  auto stage = [&](int p, int which) {
    uint8_t* buf = buf0 + which * S::kBytes;
#pragma unroll
    for (int j = 0; j < S::kLoads; ++j) {
      const int r = j * (64 / S::kSlots) + lr;           // row in the buffer
      const int pc = S::slot(r, ls);                     // piece in that slot
      const int row = min(p + r, L - 1) - span0;
      const uint32_t off = (uint32_t)row * DI + pc * 16;
      load_lds16(kb, off, buf + j * 1024);
    }
  };

  constexpr int kStep = (kThreads / 64) * kRows;
  int p0 = span0 + wave * kRows;
  int which = 0;
  if (p0 < span1) stage(p0, 0);
  for (; p0 < span1; p0 += kStep, which ^= 1) {
    const bool more = p0 + kStep < span1;
    if (more) stage(p0 + kStep, which ^ 1);
    // This buffer's loads are older than the kLoads just issued.
    if (more)
      __builtin_amdgcn_s_waitcnt(0x0F70 | (S::kLoads & 15) | ((S::kLoads >> 4) << 14));
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);
    const uint8_t* rows = buf0 + which * S::kBytes;
    // Lane (g, c) reads pieces g and g + 4 of rows 16 u + c; f(16 u + c)
    // does not depend on u.
    v8i kv[kGroups];
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
      const uint8_t* pr = rows + (u * 16 + c) * DI;
      const v4u x = *reinterpret_cast<const v4u*>(pr + S::slot(c, g) * 16);
      const v4u y = DI == 128 ? *reinterpret_cast<const v4u*>(pr + S::slot(c, g + 4) * 16)
                              : v4u{0u, 0u, 0u, 0u};
      kv[u] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                  (int)y.x, (int)y.y, (int)y.z, (int)y.w};
    }
    float mine[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) mine[j] = 0.f;
    // Group u's MFMAs are issued before group u - 1's epilogue reads its
    // results, so the matrix unit works while the epilogue runs (two sets of
    // accumulators, alternating).
    v4f accs[2][NT];
#define ESS_IDX_MFMA(U)                                                         \
  _Pragma("unroll") for (int t = 0; t < NT; ++t)                                \
    accs[(U) & 1][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(       \
        qa[t], kv[U], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
    // ReLU as a signed-integer max of the bits: a finite float is positive
    // exactly when its bits are, and -0 maps to +0 (one instruction; fmaxf
    // also quiets NaNs, which cannot occur here).
#define ESS_IDX_EPI(U)                                                          \
  {                                                                             \
    float part[MT];                                                             \
    _Pragma("unroll") for (int j = 0; j < MT; ++j) part[j] = 0.f;               \
    _Pragma("unroll") for (int t = 0; t < NT; ++t)                              \
      _Pragma("unroll") for (int r = 0; r < 4; ++r)                             \
        part[t / kTilesPerTok] = fmaf(                                          \
            wv[t][r], __int_as_float(max(__float_as_int(accs[(U) & 1][t][r]), 0)), \
            part[t / kTilesPerTok]);                                            \
    _Pragma("unroll") for (int j = 0; j < MT; ++j) {                            \
      float v = part[j];                                                        \
      v += __shfl_xor(v, 16);                                                   \
      v += __shfl_xor(v, 32);                                                   \
      if (g == (U)) mine[j] = v;   /* lane group U stores group U */            \
    }                                                                           \
  }
    ESS_IDX_MFMA(0)
#pragma unroll
    for (int u = 1; u < kGroups; ++u) {
      ESS_IDX_MFMA(u)
      ESS_IDX_EPI(u - 1)
    }
    ESS_IDX_EPI(kGroups - 1)
#undef ESS_IDX_EPI
#undef ESS_IDX_MFMA
    const int pos = p0 + g * 16 + c;
    if (pos < span1) {
#pragma unroll
      for (int j = 0; j < MT; ++j)
        scores[((size_t)b * MT + j) * L + pos] =
            pos < nv[j] ? mine[j] : -__builtin_inff();
    }
  }
}

template <int DI, int NT, int MT>
hipError_t launch_t(const ess_dims& d, const uint8_t* q, const float* w,
                    const uint8_t* k, const int32_t* n_vis, float* scores,
                    hipStream_t s, ClearSpec clr) {
  dim3 grid((d.ctx_len + kSpan - 1) / kSpan, d.batch);
  const size_t lds = (size_t)(kThreads / 64) * 2 * Stage<DI>::kBytes;
  hipError_t e = ensure_dyn_lds((const void*)index_scores_kernel<DI, NT, MT>, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((index_scores_kernel<DI, NT, MT>), grid, dim3(kThreads),
                     lds, s, q, w, k, n_vis, scores, d.ctx_len, d.idx_heads, clr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_scores(const ess_dims& d, const uint8_t* q,
                               const float* w, const uint8_t* k,
                               const int32_t* n_vis, float* scores,
                               hipStream_t s, ClearSpec clr) {
  // Shapes checked by the caller: DI in {64, 128}, H_I % 16 == 0,
  // m * H_I <= 128.
  const int rows = d.mtp * d.idx_heads;
#define ESS_IDX_CASE(DI_, NT_, MT_)                                          \
  if (d.idx_dim == DI_ && rows == NT_ * 16 && d.mtp == MT_)                 \
    return launch_t<DI_, NT_, MT_>(d, q, w, k, n_vis, scores, s, clr);
#define ESS_IDX_ROWS(DI_)                                                    \
  ESS_IDX_CASE(DI_, 1, 1) ESS_IDX_CASE(DI_, 2, 1) ESS_IDX_CASE(DI_, 3, 1)    \
  ESS_IDX_CASE(DI_, 4, 1) ESS_IDX_CASE(DI_, 5, 1) ESS_IDX_CASE(DI_, 6, 1)    \
  ESS_IDX_CASE(DI_, 7, 1) ESS_IDX_CASE(DI_, 8, 1) ESS_IDX_CASE(DI_, 2, 2)    \
  ESS_IDX_CASE(DI_, 4, 2) ESS_IDX_CASE(DI_, 6, 2) ESS_IDX_CASE(DI_, 8, 2)    \
  ESS_IDX_CASE(DI_, 3, 3) ESS_IDX_CASE(DI_, 6, 3) ESS_IDX_CASE(DI_, 4, 4)    \
  ESS_IDX_CASE(DI_, 8, 4)
  ESS_IDX_ROWS(64)
  ESS_IDX_ROWS(128)
#undef ESS_IDX_ROWS
#undef ESS_IDX_CASE
  return hipErrorInvalidValue;
}

}  // namespace ess
