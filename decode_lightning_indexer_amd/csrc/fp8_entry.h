// The 656-byte fp8 latent entry (ESS concept page, FlashTrans row: the
// host-to-device transfers move 656-byte blocks; this byte layout is the
// library's reading of that size): c_KV as 512 OCP e4m3fn bytes, four
// float32 power-of-two scales (scale j multiplies c_KV[128j, 128j + 128)),
// then k_R as 64 bf16 - 41 pieces of 16 bytes.  Dequantized values are
// e4m3 value * scale, rounded to bf16 (exact for power-of-two scales while
// the product stays in bf16's normal range).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ess {

constexpr int kEntryBytes = 656;
constexpr int kEntryPieces = kEntryBytes / 16;   // 41
constexpr int kEntryScaleOff = 512;
constexpr int kEntryRopeOff = 528;

// e4m3fn byte -> float: normal (1 + m/8) * 2^(e-7), subnormal m * 2^-9,
// exponent and mantissa all ones NaN.
__device__ __forceinline__ float e4m3fn_to_f32(unsigned x) {
  const unsigned e = (x >> 3) & 15u, m = x & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20))
              : (float)m * 0x1p-9f;
  if (e == 15u && m == 7u) v = __uint_as_float(0x7FC00000u);
  return (x & 0x80u) ? -v : v;
}

// float -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ unsigned f32_to_bf16_rne(float f) {
  const unsigned u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Eight e4m3fn bytes (little-endian in lo, hi) times sc -> eight bf16 packed
// in 16 bytes, value i in halfword i.
typedef unsigned int entry_v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ entry_v4u dequant8(unsigned lo, unsigned hi, float sc) {
  unsigned h[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = f32_to_bf16_rne(e4m3fn_to_f32((lo >> (8 * i)) & 0xFFu) * sc);
    h[4 + i] = f32_to_bf16_rne(e4m3fn_to_f32((hi >> (8 * i)) & 0xFFu) * sc);
  }
  return entry_v4u{h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                   h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

}  // namespace ess

namespace ess {

// Quantizing a bf16 latent into an entry: the block scale is the smallest
// power of two s with max|x| <= 448 s (1 for an all-zero block), and each
// c_KV value x becomes the e4m3fn code nearest x / s (ties to the even code,
// |x / s| <= 448 by the choice of s; -0 becomes +0).
__device__ __forceinline__ int entry_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int t = ilogbf(amax) - 9;                  // 448 * 2^t < amax here
  while (amax > 448.f * ldexpf(1.f, t)) ++t;
  return t;
}

__device__ __forceinline__ unsigned f32_to_e4m3fn_rne(float x) {
  const float v = fabsf(x);
  unsigned code;
  if (v < 0x1p-6f) {
    code = (unsigned)rintf(v * 512.f);       // subnormal steps of 2^-9
  } else {
    const int e = ilogbf(v);
    const unsigned m = (unsigned)rintf((ldexpf(v, -e) - 1.f) * 8.f);
    code = ((unsigned)(e + 7) << 3) + m;     // m == 8 carries into the exponent
  }
  if (code > 0x7Eu) code = 0x7Eu;
  return (x < 0.f && code != 0u) ? (code | 0x80u) : code;
}

}  // namespace ess
