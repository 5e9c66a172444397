// 8-bit floating-point KV rows (LServe blog page, section 3.2.1: the
// retrieval-head cache is stored with configurable 2-8 bit quantization).
//
// Format: OCP FP8 E4M3 codes (bias 7, 3 mantissa bits, subnormals, largest
// finite 448), converted by the gfx950 instructions v_cvt_pk_fp8_f32 (round
// to nearest even; values above 464 would give NaN, so y is clamped to +-448
// first) and v_cvt_pk_f32_fp8 (exact).  One fp32 scale per row:
// s = amax / 448 and code(x) = E4M3(x / s), both divisions correctly rounded;
// an all-zero row has s = 0 and codes 0.
//
// quantize_rows_kernel: a row of D elements is held by D/8 consecutive lanes
// (8 elements each); the row maximum is a DPP reduction over those lanes.
#include "device_common.h"
#include "launch.h"

namespace da {
namespace {

constexpr int kQuantThreads = 256;

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

template <int DT, int D>
__global__ __launch_bounds__(kQuantThreads) void quantize_rows_kernel(const void* x, uint8_t* codes,
                                                                     float* scales, long long rows) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  constexpr int RPW = kWave / LPR;
  constexpr int ROWS = (kQuantThreads / kWave) * RPW;  // rows per workgroup
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const long long row = (long long)blockIdx.x * ROWS + wave * RPW + lane / LPR;
  const int col = lane % LPR;
  const bool ok = row < rows;
  float v[8];
  if (ok) {
    if constexpr (DT == 0) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + row * D + col * 8);
      const uint4 a = src[0], b = src[1];
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __builtin_bit_cast(float, w[i]);
    } else {
      const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + row * D + col * 8);
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = group_max<LPR>(amax);  // every lane of the row takes part (rows are lane-aligned)
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
  if (ok) {
    *reinterpret_cast<uint2*>(codes + row * D + col * 8) = make_uint2((uint32_t)w0, (uint32_t)w1);
    if (col == 0) scales[row] = s;
  }
}

}  // namespace

bool quantize_supported(int dtype, int D) { return (dtype == 0 || dtype == 1) && (D == 64 || D == 128); }

hipError_t launch_quantize_rows(int dtype, int D, const void* x, uint8_t* codes, float* scales,
                                long long rows, hipStream_t stream) {
  if (rows < 1) return hipSuccess;
  const int per = (kQuantThreads / kWave) * (kWave / (D / 8));
  const long long grid = (rows + per - 1) / per;
  const dim3 g((unsigned)grid), b(kQuantThreads);
  if (dtype == 0 && D == 64) hipLaunchKernelGGL((quantize_rows_kernel<0, 64>), g, b, 0, stream, x, codes, scales, rows);
  else if (dtype == 0 && D == 128) hipLaunchKernelGGL((quantize_rows_kernel<0, 128>), g, b, 0, stream, x, codes, scales, rows);
  else if (dtype == 1 && D == 64) hipLaunchKernelGGL((quantize_rows_kernel<1, 64>), g, b, 0, stream, x, codes, scales, rows);
  else if (dtype == 1 && D == 128) hipLaunchKernelGGL((quantize_rows_kernel<1, 128>), g, b, 0, stream, x, codes, scales, rows);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

long long quantize_launch_blocks(int D, long long rows) {
  const int per = (kQuantThreads / kWave) * (kWave / (D / 8));
  return (rows + per - 1) / per;
}

}  // namespace da
