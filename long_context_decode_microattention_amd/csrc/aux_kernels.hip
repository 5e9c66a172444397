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
constexpr int kReadUnroll = 8;     // 8 KiB per wave in flight
constexpr int kReadMaxGrid = 4096;

// One workgroup per CU; every wave of the grid sweeps the buffer together:
// wave w reads the 1 KiB blocks w, w + W, w + 2W, ... (W waves in the grid,
// lane-contiguous 16-byte non-temporal loads), kReadUnroll of them in
// flight, so the reads in flight at any moment form one front across the
// buffer.  This walk measured faster than giving each workgroup its own
// contiguous chunk (7.32-7.36 vs 7.22 TB/s over 16 GiB), and waiting for the
// wave's eight loads together faster than consuming them one by one.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* __restrict__ src,
                                                                   size_t n16, uint32_t* sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const long long W = (long long)gridDim.x * (kReadThreads / kWave);
  const long long w = (long long)blockIdx.x * (kReadThreads / kWave) +
                      __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar loop
  const long long nblk = (long long)(n16 / kWave);  // whole 1 KiB blocks
  uint32_t x = 0;
  for (long long b = w; b < nblk; b += kReadUnroll * W) {
    uint4 a[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const long long bb = b + u * W;
      a[u] = bb < nblk ? load_stream16(src + bb * kWave + lane) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
  }
  // the partial last block (fewer than 64 16-byte units), by the grid's last wave
  if (w == W - 1) {
    const size_t i = (size_t)nblk * kWave + lane;
    if (i < n16) {
      const uint4 t = load_stream16(src + i);
      x ^= t.x ^ t.y ^ t.z ^ t.w;
    }
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

int stream_read_grid() { return kReadMaxGrid; }

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  int dev = 0, cus = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  const size_t n16 = bytes / 16;
  int grid = cus < 1 ? 1 : cus;
  if (grid > kReadMaxGrid) grid = kReadMaxGrid;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kReadThreads), 0, stream,
                     static_cast<const uint4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace da
