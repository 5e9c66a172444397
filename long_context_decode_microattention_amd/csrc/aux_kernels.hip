// Auxiliary kernels: device-side validation of block tables and sequence
// lengths, and a streaming-read kernel that measures the achievable HBM read
// rate.  Neither is on the attention path.
#include "device_common.h"
#include "launch.h"

namespace da {
namespace {

constexpr int kCheckThreads = 256;

// One lane per (request, logical page).  A lane that finds a violation sets
// its ballot bit; one lane per wave adds the wave's count to err[0] with a
// vector-memory atomic.
__global__ __launch_bounds__(kCheckThreads) void check_kernel(const int32_t* __restrict__ table,
                                                              const int32_t* __restrict__ lens,
                                                              int S, int P, int max_pages,
                                                              long long NP, int32_t* err) {
  const long long i = (long long)blockIdx.x * kCheckThreads + threadIdx.x;
  bool bad = false;
  if (i < (long long)S * max_pages) {
    const int s = (int)(i / max_pages);
    const int lp = (int)(i - (long long)s * max_pages);
    const int L = lens[s];
    const long long cap = (long long)max_pages * P;
    if (lp == 0 && (L < 0 || (long long)L > cap)) bad = true;
    const long long Lc = L < 0 ? 0 : ((long long)L > cap ? cap : L);
    if ((long long)lp * P < Lc) {
      const int v = table[i];
      if (v < 0 || (long long)v >= NP) bad = true;
    }
  }
  const uint64_t bal = __ballot(bad);
  if ((threadIdx.x & (kWave - 1)) == 0 && bal != 0) atomicAdd(err, (int32_t)__popcll(bal));
}

constexpr int kReadThreads = 256;
constexpr int kReadBlocksPerCU = 8;
constexpr int kReadCUs = 256;
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* __restrict__ src,
                                                                   size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    uint4 a[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) a[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // data-dependent store: the loads cannot be dropped, the store almost never happens
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}

}  // namespace

hipError_t launch_check_inputs(const int32_t* table, const int32_t* lens, int S, int P,
                               int max_pages, int64_t NP, int32_t* err, hipStream_t stream) {
  const long long n = (long long)S * max_pages;
  const long long blocks = (n + kCheckThreads - 1) / kCheckThreads;
  hipLaunchKernelGGL(check_kernel, dim3((unsigned)blocks), dim3(kCheckThreads), 0, stream, table,
                     lens, S, P, max_pages, (long long)NP, err);
  return hipGetLastError();
}

int stream_read_grid() { return kReadCUs * kReadBlocksPerCU; }

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(stream_read_grid()), dim3(kReadThreads), 0, stream,
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace da
