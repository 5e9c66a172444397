// Aggregation kernel: one workgroup per (request, query head) folds the b
// MicroAttention partials into the attention output
//   m_g = max_j m_j,  e_g = sum_j e_j exp(m_j - m_g),  out = sum_j MA_j exp(m_j - m_g) / e_g
// (Infinite-LLM page, section 方法细节, aggregation equations).  Empty
// partials (m_j = -inf) get weight exp(-inf) = 0; if all are empty, out = 0.
//
// The partial form (kPartial) stops before the division and writes the
// triple (sum_j MA_j exp(m_j - m_g), m_g, e_g) into one slot of a gather
// buffer [S, Hq, out_splits, .]: the fold an instance applies to its own
// splits before sending one triple per (request, head) back to the master.
//
// The split weights exp(m_j - m_g) are computed once per chunk of 256 splits
// into LDS; the 256 lanes then cover (split phase, dimension) pairs so that
// the loads of MA_j for many splits are in flight together.
#include "device_common.h"
#include "launch.h"

namespace da {
namespace {

constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / kWave;

template <bool kPartial>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float* __restrict__ MA,
                                                              const float* __restrict__ m,
                                                              const float* __restrict__ e,
                                                              float* __restrict__ out,
                                                              float* __restrict__ m_out,
                                                              float* __restrict__ e_out, int D,
                                                              int B, int out_splits, int slot) {
  __shared__ float s_w[kMergeThreads];
  __shared__ float s_red[kMergeWaves];
  __shared__ float s_acc[kMergeThreads];
  const size_t sh = blockIdx.x;  // s * Hq + h
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const float* mr = m + sh * B;
  const float* er = e + sh * B;
  const float* MAr = MA + sh * (size_t)B * D;
  // the output row: out [S, Hq, D], or slot `slot` of [S, Hq, out_splits, D]
  const size_t orow = kPartial ? sh * out_splits + slot : sh;

  // m_g
  float lm = neg_inf();
  for (int j = tid; j < B; j += kMergeThreads) lm = fmaxf(lm, mr[j]);
  lm = wave_max(lm);
  if (lane == 0) s_red[wave] = lm;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int w = 1; w < kMergeWaves; ++w) M = fmaxf(M, s_red[w]);
  const float Ms = (M == neg_inf()) ? 0.f : M;

  // lanes cover (phase, d): phase p sums splits p, p + NPH, ... of each chunk
  const int nph = D <= kMergeThreads ? kMergeThreads / D : 1;
  const int p = D <= kMergeThreads ? tid / D : 0;
  const int d = D <= kMergeThreads ? tid - p * D : tid;
  float acc = 0.f, le = 0.f;
  for (int jc = 0; jc < B; jc += kMergeThreads) {
    __syncthreads();  // s_w of the previous chunk is consumed; s_red is read
    const int jn = min(kMergeThreads, B - jc);
    if (tid < jn) {
      const float w = expf(mr[jc + tid] - Ms);
      s_w[tid] = w;
      le = fmaf(er[jc + tid], w, le);
    }
    __syncthreads();
    if (d < D && p < nph) {
      int jj = p;
      for (; jj + 3 * nph < jn; jj += 4 * nph) {
        const float a0 = MAr[(size_t)(jc + jj) * D + d];
        const float a1 = MAr[(size_t)(jc + jj + nph) * D + d];
        const float a2 = MAr[(size_t)(jc + jj + 2 * nph) * D + d];
        const float a3 = MAr[(size_t)(jc + jj + 3 * nph) * D + d];
        acc = fmaf(a0, s_w[jj], acc);
        acc = fmaf(a1, s_w[jj + nph], acc);
        acc = fmaf(a2, s_w[jj + 2 * nph], acc);
        acc = fmaf(a3, s_w[jj + 3 * nph], acc);
      }
      for (; jj < jn; jj += nph) acc = fmaf(MAr[(size_t)(jc + jj) * D + d], s_w[jj], acc);
    }
  }

  // e_g
  le = wave_sum(le);
  __syncthreads();
  if (lane == 0) s_red[wave] = le;
  s_acc[tid] = acc;
  __syncthreads();
  float eg = 0.f;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) eg += s_red[w];
  if (kPartial && tid == 0) {
    m_out[orow] = M;
    e_out[orow] = eg;
  }

  if (D <= kMergeThreads) {
    if (tid < D) {
      float total = 0.f;
      for (int q = 0; q < nph; ++q) total += s_acc[q * D + tid];
      out[orow * D + tid] = kPartial ? total : (eg > 0.f ? total / eg : 0.f);
    }
  } else {
    // D > 256: every lane owns a strided set of dimensions (not used by the
    // micro-attention kernels, which produce D = 64 or 128)
    for (int dd = tid; dd < D; dd += kMergeThreads) {
      float t = 0.f;
      for (int j = 0; j < B; ++j) t = fmaf(MAr[(size_t)j * D + dd], expf(mr[j] - Ms), t);
      out[orow * D + dd] = kPartial ? t : (eg > 0.f ? t / eg : 0.f);
    }
  }
}

// Folds the page-range chunks of each split back into the split's triple
// (the same aggregation rule, keeping the triple form): one wave per
// (request, head, split).  Lane c holds chunk c's (m, e) (at most 64
// chunks), so the maximum and the sum are wave reductions; the chunk weights
// go through LDS, and each lane has the loads of its dimension for
// kCombineBatch chunks in flight before it accumulates them.
constexpr int kCombineBatch = 16;

__global__ __launch_bounds__(kWave) void combine_kernel(const float* __restrict__ cMA,
                                                        const float* __restrict__ cm,
                                                        const float* __restrict__ ce,
                                                        float* __restrict__ MA,
                                                        float* __restrict__ m,
                                                        float* __restrict__ e, int chunks, int D) {
  __shared__ float s_w[kWave];
  const size_t o = blockIdx.x;
  const int lane = threadIdx.x;
  const float* MAr = cMA + o * (size_t)chunks * D;
  const bool own = lane < chunks;
  const float mc = own ? cm[o * chunks + lane] : neg_inf();
  const float ec = own ? ce[o * chunks + lane] : 0.f;
  const float M = wave_max(mc);
  const float Ms = (M == neg_inf()) ? 0.f : M;
  const float w = own ? expf(mc - Ms) : 0.f;  // 0 for an empty chunk (mc = -inf)
  const float eg = wave_sum(ec * w);
  s_w[lane] = w;
  __syncthreads();
  for (int d = lane; d < D; d += kWave) {
    float acc = 0.f;
    int c = 0;
    for (; c + kCombineBatch <= chunks; c += kCombineBatch) {
      float x[kCombineBatch];
#pragma unroll
      for (int u = 0; u < kCombineBatch; ++u) x[u] = MAr[(size_t)(c + u) * D + d];
#pragma unroll
      for (int u = 0; u < kCombineBatch; ++u) acc = fmaf(x[u], s_w[c + u], acc);
    }
    for (; c < chunks; ++c) acc = fmaf(MAr[(size_t)c * D + d], s_w[c], acc);
    MA[o * D + d] = acc;
  }
  if (lane == 0) {
    m[o] = M;
    e[o] = eg;
  }
}

__global__ void queue_reset_kernel(int* queue) {
  if (threadIdx.x < kQueues) queue[threadIdx.x * kQueueStride] = 0;
}

__global__ __launch_bounds__(256) void zero_ints_kernel(int* p, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_queue_reset(int* queue, hipStream_t stream) {
  hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(kWave), 0, stream, queue);
  return hipGetLastError();
}

hipError_t launch_zero_ints(int* p, long long n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_ints_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_combine(const float* cMA, const float* cm, const float* ce, float* MA, float* m,
                          float* e, long long n, int chunks, int D, hipStream_t stream) {
  if (chunks < 1 || chunks > kWave) return hipErrorInvalidValue;  // one lane per chunk
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)n), dim3(kWave), 0, stream, cMA, cm, ce, MA, m,
                     e, chunks, D);
  return hipGetLastError();
}

hipError_t launch_merge(const float* MA, const float* m, const float* e, float* out, int S, int Hq,
                        int D, int B, hipStream_t stream) {
  const long long n = (long long)S * Hq;
  hipLaunchKernelGGL(merge_kernel<false>, dim3((unsigned)n), dim3(kMergeThreads), 0, stream, MA, m,
                     e, out, nullptr, nullptr, D, B, 1, 0);
  return hipGetLastError();
}

hipError_t launch_merge_partials(const float* MA, const float* m, const float* e, float* MA_out,
                                 float* m_out, float* e_out, int S, int Hq, int D, int B,
                                 int out_splits, int slot, hipStream_t stream) {
  const long long n = (long long)S * Hq;
  hipLaunchKernelGGL(merge_kernel<true>, dim3((unsigned)n), dim3(kMergeThreads), 0, stream, MA, m,
                     e, MA_out, m_out, e_out, D, B, out_splits, slot);
  return hipGetLastError();
}

}  // namespace da
