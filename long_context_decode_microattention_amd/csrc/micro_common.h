// Pieces shared by the MicroAttention kernels: work-item decoding (with the
// optional cut of a split into page-range chunks), kept-page compaction into
// LDS, and the end-of-item combine of the four waves' partial triples.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace da {

constexpr int kMicroThreads = 256;
constexpr int kMicroWaves = kMicroThreads / kWave;
constexpr int kPageCap = 1024;  // kept pages staged in LDS per batch
constexpr int kSlab = 16;       // tokens per slab

// One work item: (request s, KV head kvh, split j, piece c).  A split is the
// token range [t0, t1) (split bounds intersected with [0, L_s)) on logical
// pages [pa, pb); piece c of `chunks` takes the logical pages
// [scan0, scan1) = the c-th equal share of [pa, pb), and within them the
// pages the block mask keeps.
struct Item {
  int s, kvh, j, c;
  int t0, t1;        // split token range (empty if t0 >= t1)
  int scan0, scan1;  // logical pages of this piece
  const uint8_t* mrow;  // block-mask row of (s, kvh), or null
};

__device__ __forceinline__ Item plan_item(const MicroParams& p, int x) {
  Item it;
  it.c = x % p.chunks;
  x /= p.chunks;
  it.j = x % p.max_splits;
  x /= p.max_splits;
  it.kvh = x % p.Hkv;
  it.s = x / p.Hkv;
  const int P = p.P;
  it.mrow = p.mask ? p.mask + ((size_t)it.s * p.Hkv + it.kvh) * p.max_pages : nullptr;
  int Ls = p.lens[it.s];
  Ls = max(0, min(Ls, p.max_pages * P));
  const int32_t* sb = p.bounds + ((size_t)it.s * (p.bounds_per_head ? p.Hkv : 1) +
                                  (p.bounds_per_head ? it.kvh : 0)) *
                                     (size_t)(p.max_splits + 1);
  it.t0 = max(sb[it.j], 0);
  it.t1 = min(sb[it.j + 1], Ls);
  it.scan0 = it.scan1 = 0;
  if (it.t0 < it.t1) {
    const int pa = it.t0 / P, pb = (it.t1 + P - 1) / P;
    const long long n = pb - pa;
    it.scan0 = pa + (int)((n * it.c) / p.chunks);
    it.scan1 = pa + (int)((n * (it.c + 1)) / p.chunks);
  }
  return it;
}

// The fused-merge arguments, copied to LDS once per workgroup before the
// first item and read back at the end of each item, so that they hold no
// scalar registers across the slab loop.  The fused merge is a separate
// kernel instance (template flag kFused): compiled into every instance, its
// code raised the register allocation of the slab loop by ~20 VGPRs even
// where it never runs (one wave per SIMD less for the vector kernel).
struct FusedArgs {
  int* group_count;
  float* out;
};
static __shared__ FusedArgs s_fused;

// Runs body(x) for every work item x this workgroup owns (kFused: the
// kernel instance with the fused merge): item blockIdx.x
// for a one-per-item launch, or, for a persistent launch, items claimed from
// p.queue `grab` at a time in increasing order until none are left.  The
// next claim is issued before the current items are processed, so its
// latency is hidden.  body may use LDS and barriers; every lane calls it with
// the same x.
template <bool kFused, class Body>
__device__ __forceinline__ void for_each_item(const MicroParams& p, int* s_claim, Body&& body) {
  if constexpr (kFused) {
    if (threadIdx.x == 0) s_fused = FusedArgs{p.group_count, p.out};  // read after later barriers
  }
  if (p.queue == nullptr) {
    body((int)blockIdx.x);
    return;
  }
  const int tid = threadIdx.x;
  if (tid == 0) *s_claim = atomicAdd(p.queue, p.grab);
  __syncthreads();
  int x0 = __builtin_amdgcn_readfirstlane(*s_claim);
  while (x0 >= 0 && x0 < p.n_items) {  // a counter not reset to 0 ends the loop
    int next = 0;
    if (tid == 0) next = atomicAdd(p.queue, p.grab);
    const int x1 = min(x0 + p.grab, p.n_items);
    for (int x = x0; x < x1; ++x) {
      body(x);
      __syncthreads();  // the item's LDS (page list, combine) is free again
    }
    if (tid == 0) *s_claim = next;
    __syncthreads();
    x0 = __builtin_amdgcn_readfirstlane(*s_claim);
  }
}

// Compacts the kept pages of [base, min(base + kPageCap, lp1)) into LDS
// (physical page ids and logical page ids, in logical order) with wave
// ballots; returns the count.  Every thread of the workgroup must call it.

__device__ __forceinline__ int compact_pages(int base, int lp1, const uint8_t* mrow,
                                             const int32_t* trow, int* s_phys, int* s_lp,
                                             int* s_cnt) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  int nk = 0;
  const int span = min(kPageCap, lp1 - base);
  for (int r = 0; r < span; r += kMicroThreads) {
    const int lp = base + r + tid;
    const bool keep = lp < lp1 && (mrow == nullptr || mrow[lp] != 0);
    const uint64_t bal = __ballot(keep);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = nk;
    for (int w = 0; w < wave; ++w) off += s_cnt[w];
    if (keep) {
      s_phys[off + pre] = trow[lp];
      s_lp[off + pre] = lp;
    }
    nk += s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
    __syncthreads();
  }
  // the count is the same in every lane; saying so keeps the slab loop scalar
  return __builtin_amdgcn_readfirstlane(nk);
}

// LDS for the end-of-item combine.
template <int G, int D>
struct FinishLds {
  float acc[kMicroWaves][G][D];
  float m[kMicroWaves][G];
  float e[kMicroWaves][G];
  int last;  // fused merge: this item completed its group
};

// Device-scope (agent) relaxed store and load: coherent across the XCDs'
// L2 caches by themselves, so partials written by one workgroup can be read
// by another without cache-wide fences.
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this wave's vector memory operations (its stores) completed:
// s_waitcnt vmcnt(0), the other counters left unconstrained.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Fused merge.  Called by every thread after the item's partials are
// written.  The partials are released to device scope and the group's
// counter counted up; the item that brings it to max_splits * chunks folds
// all partials of the group's G query heads with the aggregation rule of
// the merge kernel (m_g = max m_j, w_j = exp(m_j - m_g), e_g = sum e_j w_j,
// out = sum MA_j w_j / e_g, out = 0 when every partial is empty) and sets
// the counter back to zero for the next call.  No workgroup waits for
// another: only the last arrival does more work.
template <int G, int D>
__device__ __forceinline__ void merge_group(const MicroParams& p, const Item& it, FinishLds<G, D>& L) {
  static_assert(kMicroThreads % D == 0 && G * D * kMicroWaves >= kMicroThreads, "merge scratch");
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = p.max_splits * p.chunks;
  int* count = s_fused.group_count + (size_t)it.s * p.Hkv + it.kvh;
  // The partials were written as device-scope atomic stores (sc1: made
  // coherent across the XCDs' L2 caches by the access itself, as the
  // compiler's memory model implements monotonic device-scope atomics) and
  // are read back the same way; waiting until they have completed orders
  // them before the counter.  A device-scope fence, or an acquire-release
  // counter update, writes back and invalidates a whole L2 per item:
  // measured 0.2-0.35 us per item with the fence in every thread, and with
  // the acquire-release update in one thread C2 366 us against 194 us and
  // C3 2.93 ms against 1.0 ms.
  wait_stores();
  __syncthreads();
  if (tid == 0) L.last = atomicAdd(count, 1) == n - 1;
  __syncthreads();
  if (!L.last) return;
  const size_t h0 = (size_t)it.s * p.Hq + it.kvh * G;  // first query head of the group
  constexpr int SCR = kMicroWaves * G * D;              // floats of scratch in L.acc
  constexpr int GD = G * D;
  float* sw = &L.acc[0][0][0];
  if (2 * G * n <= SCR) {
    // m and e of every partial of the group into LDS in one pass (the
    // group's heads are consecutive, so its partials are one run)
    for (int x = tid; x < G * n; x += kMicroThreads) {
      sw[x] = load_dev(p.m + h0 * n + x);
      sw[G * n + x] = load_dev(p.e + h0 * n + x);
    }
    __syncthreads();
    // per head (one wave each): m_g, the weights exp(m_i - m_g) in place of
    // the m_i, and e_g
    for (int g = wave; g < G; g += kMicroWaves) {
      float lm = neg_inf();
      for (int i = lane; i < n; i += kWave) lm = fmaxf(lm, sw[g * n + i]);
      const float M = wave_max(lm);
      const float Ms = (M == neg_inf()) ? 0.f : M;
      float le = 0.f;
      for (int i = lane; i < n; i += kWave) {
        const float w = expf(sw[g * n + i] - Ms);
        le = fmaf(sw[G * n + g * n + i], w, le);
        sw[g * n + i] = w;
      }
      le = wave_sum(le);
      if (lane == 0) L.e[0][g] = le;
    }
    __syncthreads();
    // value sums of the G * D outputs, each split into phs phases over the
    // partials (all threads busy), 8 loads in flight per thread; the phase
    // sums go where the e_i were
    const int phs = max(1, min(kMicroThreads / GD, (SCR - G * n) / GD));
    float* red = sw + G * n;
    for (int t = tid; t < phs * GD; t += kMicroThreads) {
      const int o = t % GD, ph = t / GD;
      const int g = o / D, d = o - g * D;
      const float* MAr = p.MA + (h0 + g) * n * D + d;
      const float* w = sw + g * n;
      float acc = 0.f;
      int i = ph;
      for (; i + 7 * phs < n; i += 8 * phs) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = load_dev(MAr + (size_t)(i + u * phs) * D);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = fmaf(x[u], w[i + u * phs], acc);
      }
      for (; i < n; i += phs) acc = fmaf(load_dev(MAr + (size_t)i * D), w[i], acc);
      if (phs == 1) {
        const float eg = L.e[0][g];
        s_fused.out[(h0 + g) * D + d] = eg > 0.f ? acc / eg : 0.f;
      } else {
        red[t] = acc;
      }
    }
    if (phs > 1) {
      __syncthreads();
      for (int o = tid; o < GD; o += kMicroThreads) {
        float total = 0.f;
        for (int q = 0; q < phs; ++q) total += red[q * GD + o];
        const int g = o / D;
        const float eg = L.e[0][g];
        s_fused.out[(h0 + g) * D + (o - g * D)] = eg > 0.f ? total / eg : 0.f;
      }
    }
  } else {
    // many partials (more than 2 D per head): head by head, in phases of D
    constexpr int PH = kMicroThreads / D;
    const int d = tid % D;
    const int ph = tid / D;
    float* red = sw;  // kMicroThreads floats
    for (int g = 0; g < G; ++g) {
      const size_t h = h0 + g;
      const float* mr = p.m + h * n;
      const float* er = p.e + h * n;
      const float* MAr = p.MA + h * n * D;
      float lm = neg_inf();
      for (int i = tid; i < n; i += kMicroThreads) lm = fmaxf(lm, load_dev(mr + i));
      lm = wave_max(lm);
      if (lane == 0) L.m[wave][g] = lm;
      __syncthreads();
      float M = L.m[0][g];
#pragma unroll
      for (int w = 1; w < kMicroWaves; ++w) M = fmaxf(M, L.m[w][g]);
      const float Ms = (M == neg_inf()) ? 0.f : M;
      float le = 0.f;
      for (int i = tid; i < n; i += kMicroThreads)
        le = fmaf(load_dev(er + i), expf(load_dev(mr + i) - Ms), le);
      le = wave_sum(le);
      if (lane == 0) L.e[wave][g] = le;
      float acc = 0.f;
      for (int i = ph; i < n; i += PH)
        acc = fmaf(load_dev(MAr + (size_t)i * D + d), expf(load_dev(mr + i) - Ms), acc);
      red[tid] = acc;
      __syncthreads();
      if (tid < D) {
        float total = 0.f;
#pragma unroll
        for (int q = 0; q < PH; ++q) total += red[q * D + tid];
        float eg = 0.f;
#pragma unroll
        for (int w = 0; w < kMicroWaves; ++w) eg += L.e[w][g];
        s_fused.out[h * D + tid] = eg > 0.f ? total / eg : 0.f;
      }
      __syncthreads();
    }
  }
  if (tid == 0) *count = 0;
}

// Combines the four waves' triples and writes the item's partials.  Each
// wave supplies, per head g: raw-dot maximum wm[g] and exp-sum we[g] (valid
// in every lane) and, in the lanes of its first row (lane < LPT), the value
// sums acc[g][k] for dimensions lane*EPL + k.  Output index
// ((s*Hq + h)*max_splits + j)*chunks + c.
template <int G, int D, int LPT, int EPL, bool kFused>
__device__ __forceinline__ void finish_item(const MicroParams& p, const Item& it, FinishLds<G, D>& L,
                                            const float (&wm)[G], const float (&we)[G],
                                            const float (&acc)[G][EPL], float c) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  if (lane < LPT) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int k = 0; k < EPL; ++k) L.acc[wave][g][lane * EPL + k] = acc[g][k];
      if (lane == 0) {
        L.m[wave][g] = wm[g];
        L.e[wave][g] = we[g];
      }
    }
  }
  __syncthreads();
  const int h0 = it.kvh * G;
  for (int idx = tid; idx < G * D; idx += kMicroThreads) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = L.m[0][g];
#pragma unroll
    for (int w = 1; w < kMicroWaves; ++w) M = fmaxf(M, L.m[w][g]);
    const float Ms = (M == neg_inf()) ? 0.f : M;
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kMicroWaves; ++w) {
      const float f = fast_exp2((L.m[w][g] - Ms) * c);
      num = fmaf(L.acc[w][g][d], f, num);
      den = fmaf(L.e[w][g], f, den);
    }
    const size_t o = ((size_t)(it.s * p.Hq + h0 + g) * p.max_splits + it.j) * p.chunks + it.c;
    if constexpr (kFused) {  // read by another workgroup of the same launch
      store_dev(p.MA + o * D + d, num);
      if (d == 0) {
        store_dev(p.m + o, M * p.scale);
        store_dev(p.e + o, den);
      }
    } else {
      p.MA[o * D + d] = num;
      if (d == 0) {
        p.m[o] = M * p.scale;
        p.e[o] = den;
      }
    }
  }
  if constexpr (kFused) merge_group<G, D>(p, it, L);
}

// Dynamic LDS that caps a kernel at `wg` resident workgroups per CU (0 = no
// cap): each workgroup is padded to just over 1/(wg+1) of the CU's LDS.  On
// gfx950 fewer, deeper streams per CU read HBM faster than many shallow ones.
inline size_t occupancy_lds(const void* kernel, int wg) {
  if (wg <= 0) return 0;
  int dev = 0, per_cu = 0, per_block = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
          hipSuccess ||
      hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return 0;
  hipFuncAttributes attr;
  if (hipFuncGetAttributes(&attr, kernel) != hipSuccess) return 0;
  const size_t want = ((size_t)per_cu / (wg + 1) / 1024 + 1) * 1024;  // > per_cu / (wg + 1)
  if (want * wg > (size_t)per_cu || want > (size_t)per_block || want <= attr.sharedSizeBytes)
    return 0;
  return want - attr.sharedSizeBytes;
}

// Workgroups of `kernel` that fit on the device at once with `lds` bytes of
// dynamic LDS each (the grid of a persistent launch).
inline int resident_slots(const void* kernel, size_t lds) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kMicroThreads, lds) !=
          hipSuccess)
    return 0;
  return cus * per_cu;
}

// A grid this many times larger than the resident slots goes persistent.
constexpr long long kPersistentFactor = 8;

// Launches a MicroAttention kernel.  Normally one workgroup per item: the
// hardware dispatcher keeps the slots full.  When the grid is far larger
// than the resident slots (many small or empty items, as in ragged batches)
// and p.queue provides a counter, the in-order, XCD-round-robin dispatch
// itself becomes the bottleneck; then the launch is persistent: one
// workgroup per resident slot, each claiming items from the counter in
// batches small enough that the tail stays short.
template <class Kernel>
hipError_t launch_micro_kernel(Kernel kernel, int wg_per_cu, MicroParams p, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(kernel);
  const size_t lds = occupancy_lds(fn, wg_per_cu);
  long long grid = p.n_items;
  if (p.queue != nullptr) {
    const int slots = resident_slots(fn, lds);
    const bool go = p.schedule == 2 || (p.schedule == 0 && p.n_items > kPersistentFactor * slots);
    if (slots > 0 && go) {
      const hipError_t err = launch_queue_reset(p.queue, stream);
      if (err != hipSuccess) return err;
      grid = slots;
      const long long per = (long long)p.n_items / ((long long)slots * 16);
      p.grab = (int)(per < 1 ? 1 : (per > 64 ? 64 : per));
    } else {
      p.queue = nullptr;
    }
  }
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kMicroThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace da
