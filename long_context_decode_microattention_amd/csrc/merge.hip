// Aggregation kernel: one wave per (request, query head) folds the b
// MicroAttention partials into the attention output
//   m_g = max_j m_j,  e_g = sum_j e_j exp(m_j - m_g),  out = sum_j MA_j exp(m_j - m_g) / e_g
// (Infinite-LLM page, section 方法细节, aggregation equations).  Empty
// partials (m_j = -inf) get weight exp(-inf) = 0; if all are empty, out = 0.
#include "device_common.h"
#include "launch.h"

namespace da {
namespace {

__global__ __launch_bounds__(kWave) void merge_kernel(const float* __restrict__ MA,
                                                      const float* __restrict__ m,
                                                      const float* __restrict__ e,
                                                      float* __restrict__ out, int D, int B) {
  const size_t sh = blockIdx.x;  // s * Hq + h
  const int lane = threadIdx.x;
  const float* mr = m + sh * B;
  const float* er = e + sh * B;
  const float* MAr = MA + sh * (size_t)B * D;

  float M = neg_inf();
  for (int j = 0; j < B; ++j) M = fmaxf(M, mr[j]);
  const float Ms = (M == neg_inf()) ? 0.f : M;

  float eg = 0.f;
  for (int j = 0; j < B; ++j) eg = fmaf(er[j], expf(mr[j] - Ms), eg);

  for (int d = lane; d < D; d += kWave) {
    float acc = 0.f;
    for (int j = 0; j < B; ++j) acc = fmaf(MAr[(size_t)j * D + d], expf(mr[j] - Ms), acc);
    out[sh * D + d] = eg > 0.f ? acc / eg : 0.f;
  }
}

}  // namespace

hipError_t launch_merge(const float* MA, const float* m, const float* e, float* out, int S, int Hq,
                        int D, int B, hipStream_t stream) {
  const long long n = (long long)S * Hq;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)n), dim3(kWave), 0, stream, MA, m, e, out, D, B);
  return hipGetLastError();
}

}  // namespace da
