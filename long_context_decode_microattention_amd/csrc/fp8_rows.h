// Quantization of D-wide rows to 8-bit OCP FP8 E4M3 or 4-bit OCP FP4 E2M1
// codes with one fp32 scale per row, shared by the bulk row quantizer and the
// decode-time append.  8 bits: s = amax / 448 and code(x) = E4M3(x / s),
// both divisions correctly rounded; y is clamped to +-448 first
// (v_cvt_pk_fp8_f32 rounds to nearest even in range and gives NaN above
// 464).  4 bits: s = amax / 6 and code(x) = the E2M1 value nearest to x / s
// (|y| clamped to 6, ties to mantissa bit 0, the sign of y kept), two codes
// per byte, element 2i in the low nibble.  An all-zero row has s = 0 and
// codes 0.  A row is held by D/8 consecutive lanes, 8 elements each.
#pragma once

#include "device_common.h"

namespace da {

template <int N>
__device__ __forceinline__ float group_max(float x) {
  static_assert(N == 8 || N == 16, "group size");
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  if constexpr (N == 16) x = fmaxf(x, dpp<kDppRowMirror>(x));
  return x;
}

// Two fp32 values to two E4M3 codes in the low (HI = false) or high half of
// `old`, after clamping to the finite range.
template <bool HI>
__device__ __forceinline__ int pack_fp8(float a, float b, int old) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// 8 elements of 16 (bf16) or 32 (fp32) bytes at p -> floats.
template <int DT>
__device__ __forceinline__ void load8(const void* p, float (&v)[8]) {
  if constexpr (DT == 0) {
    const uint4 a = reinterpret_cast<const uint4*>(p)[0], b = reinterpret_cast<const uint4*>(p)[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __builtin_bit_cast(float, w[i]);
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  }
}

// This lane's 8 codes (two words) and the row scale.  Every lane of the row's
// LPR-lane group must call it (the row maximum is a DPP reduction); lanes of
// a row that does not exist pass zeros.
template <int LPR>
__device__ __forceinline__ uint2 quantize8(const float (&v)[8], float& scale) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = group_max<LPR>(amax);
  const float s = __fdiv_rn(amax, 448.f);
  int w0 = 0, w1 = 0;
  if (s > 0.f) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = __fdiv_rn(v[i], s);
    w0 = pack_fp8<false>(y[0], y[1], 0);
    w0 = pack_fp8<true>(y[2], y[3], w0);
    w1 = pack_fp8<false>(y[4], y[5], 0);
    w1 = pack_fp8<true>(y[6], y[7], w1);
  }
  scale = s;
  return make_uint2((uint32_t)w0, (uint32_t)w1);
}

// Magnitude code (0-7) of the E2M1 value nearest to a >= 0, whose grid is
// 0, 0.5, 1, 1.5, 2, 3, 4, 6: a compare per midpoint, each tie going to the
// neighbour with mantissa bit 0 (even code), everything above 5 to 6 (the
// clamp).
__device__ __forceinline__ uint32_t e2m1_magnitude(float a) {
  return a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
       : a <= 2.5f  ? 4u : a < 3.5f  ? 5u : a <= 5.f   ? 6u : 7u;
}

// This lane's 8 elements as eight E2M1 codes in one word (element i in bits
// 4i + 3 .. 4i) and the row scale; called like quantize8.
template <int LPR>
__device__ __forceinline__ uint32_t quantize4(const float (&v)[8], float& scale) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = group_max<LPR>(amax);
  const float s = __fdiv_rn(amax, 6.f);
  uint32_t w = 0;
  if (s > 0.f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = __fdiv_rn(v[i], s);
      const uint32_t sign = (__builtin_bit_cast(uint32_t, y) >> 31) << 3;
      w |= (e2m1_magnitude(fabsf(y)) | sign) << (4 * i);
    }
  }
  scale = s;
  return w;
}

}  // namespace da
