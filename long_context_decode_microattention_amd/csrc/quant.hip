// 8- and 4-bit floating-point KV rows (LServe blog page, section 3.2.1: the
// retrieval-head cache is stored with configurable 2-8 bit quantization, the
// streaming-head cache in 4 bits).  4-bit rows: OCP FP4 E2M1 codes, s = amax
// / 6, nearest value with ties to mantissa bit 0, two codes per byte
// (fp8_rows.h).
//
// 8-bit format: OCP FP8 E4M3 codes (bias 7, 3 mantissa bits, subnormals, largest
// finite 448), converted by the gfx950 instructions v_cvt_pk_fp8_f32 (round
// to nearest even; values above 464 would give NaN, so y is clamped to +-448
// first) and v_cvt_pk_f32_fp8 (exact).  One fp32 scale per row:
// s = amax / 448 and code(x) = E4M3(x / s), both divisions correctly rounded;
// an all-zero row has s = 0 and codes 0.
//
// quantize_rows_kernel: a row of D elements is held by D/8 consecutive lanes
// (8 elements each); the row maximum is a DPP reduction over those lanes
// (fp8_rows.h, shared with the decode-time append of 8-bit pages).
#include "fp8_rows.h"
#include "launch.h"

namespace da {
namespace {

constexpr int kQuantThreads = 256;

template <int DT, int D, int BITS>
__global__ __launch_bounds__(kQuantThreads) void quantize_rows_kernel(const void* x, uint8_t* codes,
                                                                     float* scales, long long rows) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  constexpr int RB = D * BITS / 8;  // code bytes per row
  constexpr int RPW = kWave / LPR;
  constexpr int ROWS = (kQuantThreads / kWave) * RPW;  // rows per workgroup
  constexpr int ES = DT == 0 ? 4 : 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const long long row = (long long)blockIdx.x * ROWS + wave * RPW + lane / LPR;
  const int col = lane % LPR;
  const bool ok = row < rows;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (ok) load8<DT>(static_cast<const char*>(x) + (row * D + col * 8) * ES, v);
  float s;
  if constexpr (BITS == 8) {
    const uint2 c = quantize8<LPR>(v, s);  // every lane of the row takes part
    if (ok) *reinterpret_cast<uint2*>(codes + row * RB + col * 8) = c;
  } else {
    const uint32_t c = quantize4<LPR>(v, s);
    if (ok) *reinterpret_cast<uint32_t*>(codes + row * RB + col * 4) = c;
  }
  if (ok && col == 0) scales[row] = s;
}

}  // namespace

bool quantize_supported(int dtype, int D) { return (dtype == 0 || dtype == 1) && (D == 64 || D == 128); }

template <int BITS>
hipError_t launch_rows(int dtype, int D, const void* x, uint8_t* codes, float* scales,
                       long long rows, hipStream_t stream) {
  const dim3 g((unsigned)quantize_launch_blocks(D, rows)), b(kQuantThreads);
  if (dtype == 0 && D == 64) hipLaunchKernelGGL((quantize_rows_kernel<0, 64, BITS>), g, b, 0, stream, x, codes, scales, rows);
  else if (dtype == 0 && D == 128) hipLaunchKernelGGL((quantize_rows_kernel<0, 128, BITS>), g, b, 0, stream, x, codes, scales, rows);
  else if (dtype == 1 && D == 64) hipLaunchKernelGGL((quantize_rows_kernel<1, 64, BITS>), g, b, 0, stream, x, codes, scales, rows);
  else if (dtype == 1 && D == 128) hipLaunchKernelGGL((quantize_rows_kernel<1, 128, BITS>), g, b, 0, stream, x, codes, scales, rows);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quantize_rows(int dtype, int D, int bits, const void* x, uint8_t* codes,
                                float* scales, long long rows, hipStream_t stream) {
  if (rows < 1) return hipSuccess;
  if (bits == 8) return launch_rows<8>(dtype, D, x, codes, scales, rows, stream);
  if (bits == 4) return launch_rows<4>(dtype, D, x, codes, scales, rows, stream);
  return hipErrorInvalidValue;
}

long long quantize_launch_blocks(int D, long long rows) {
  const int per = (kQuantThreads / kWave) * (kWave / (D / 8));
  return rows / per + (rows % per != 0 ? 1 : 0);  // no overflow near the int64 limit
}

}  // namespace da
