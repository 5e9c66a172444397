// Device helpers shared by the gfx950 kernels: wave64 cross-lane reductions
// and bf16 handling.  Internal to libda.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// DPP control words (GCN/CDNA data-parallel primitives on 16-lane rows).
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each 8-lane half row
constexpr int kDppRowMirror = 0x140;  // lane i <-> 15-i inside each 16-lane row

// Every permutation used here reads a lane of the same row, so no lane takes
// the bound-control fill; a plain DPP move with that fill lets the compiler
// fold the permutation into the instruction that consumes it (one
// v_add_f32_dpp / v_max_f32_dpp instead of two moves and the operation).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  const int xi = __builtin_bit_cast(int, x);
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(xi, CTRL, 0xF, 0xF, true));
}

// True in every lane if `c` holds in any lane (a scalar, wave-uniform value:
// branches on it skip code instead of masking it).
__device__ __forceinline__ bool wave_any(bool c) { return __builtin_amdgcn_ballot_w64(c) != 0; }

// Sum over aligned groups of N consecutive lanes (N = 2, 4, 8, 16 or 32);
// every lane of the group receives the group total.  The first quad step
// sums lane pairs; after the two quad steps each
// lane holds its quad's sum; the half-row mirror pairs every lane with a lane
// of the other quad of its 8-lane half, the row mirror with a lane of the
// other half of its 16-lane row; a 32-lane group finishes with an exchange
// across rows.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16 || N == 32, "group size");
  x += dpp<kDppQuadXor1>(x);
  if constexpr (N == 2) return x;
  x += dpp<kDppQuadXor2>(x);
  if constexpr (N == 4) return x;
  x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (N == 32) x += __shfl_xor(x, 16, kWave);
  return x;
}

// Maximum and sum over the 64 lanes of a wave; every lane receives the result.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// bf16 pair packed in a 32-bit word -> the two float values (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// a.x*b.x + a.y*b.y + c for bf16 pairs, accumulated in fp32 (v_dot2 on gfx950).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two OCP E4M3 codes of a word (bytes 0-1, or 2-3 when HI) -> a bf16 pair
// in one word, exactly (every E4M3 value is a bf16 value): the scaled
// conversion v_cvt_scalef32_pk_bf16_fp8 with scale 1.  Its packed result is
// read as one 32-bit word (checked on gfx950 for all 256 codes).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}

// Four OCP E4M3 codes packed in a word (byte i = element i) -> four floats,
// exactly (v_cvt_pk_f32_fp8 on gfx950).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* out) {
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  out[0] = lo.x;
  out[1] = lo.y;
  out[2] = hi.x;
  out[3] = hi.y;
}

// Two OCP FP4 E2M1 codes, the low and high nibble of byte B of a word (the
// row elements 2B and 2B + 1 of the word's eight) -> a bf16 pair in one word,
// exactly (every E2M1 value is a bf16 value): v_cvt_scalef32_pk_bf16_fp4
// with scale 1.
template <int B>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B));
}

// Eight E2M1 codes packed in a word (element i in bits 4i + 3 .. 4i) ->
// eight floats, exactly (v_cvt_scalef32_pk_f32_fp4 with scale 1, one byte at
// a time).
__device__ __forceinline__ void fp4x8_to_f32(uint32_t w, float* out) {
  const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  out[0] = a.x;
  out[1] = a.y;
  out[2] = b.x;
  out[3] = b.y;
  out[4] = c.x;
  out[5] = c.y;
  out[6] = d.x;
  out[7] = d.y;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load with the non-temporal hint: data read once (the KV stream)
// bypasses cache allocation, which sustains a markedly higher HBM read rate
// on gfx950 than a plain load.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// 16-byte store with the non-temporal hint, for results written once and not
// read back by the same kernel.  Where a kernel's writes share HBM with a
// heavy read stream this is markedly cheaper than a plain store (the page
// statistics kernel: 10% less time for 11% of its bytes written).
__device__ __forceinline__ void store_stream16(void* p, const uint4& v) {
  const u32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
}

}  // namespace da
