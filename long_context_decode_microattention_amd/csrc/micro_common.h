// Pieces shared by the MicroAttention kernels: work-item decoding (with the
// optional cut of a split into pieces of its kept pages), kept-page
// compaction into LDS, and the end-of-item combine of the four waves' partial
// triples.
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
// pages [pa, pb); piece c takes a contiguous run of the split's kept pages
// (plan_piece).
struct Item {
  int s, kvh, j, c;
  int t0, t1;        // split token range (empty if t0 >= t1)
  int pa, pb;        // logical pages of the split
  const uint8_t* mrow;  // block-mask row of (s, kvh), or null
};

// Items are numbered piece slowest: x = c * (S * Hkv * b) + (s * Hkv + kvh) * b
// + j.  Every split has a non-empty first piece, and the later pieces are
// empty for splits with few kept pages, so the non-empty items come first
// and form one run.  Empty items scattered through the grid at a regular
// stride (the piece numbered fastest, 4 pieces, block-sparse splits with one
// piece) serialised the long items: the hardware hands workgroups to the 8
// XCDs round-robin by index, and inside each XCD the long items did not fill
// the slots the short ones left (a per-workgroup trace of XCC id and
// real-time clock: 64 long items per XCD, 221 us each, ran in about four
// rounds, 971 us, against 343 us for the same items numbered in one run).
// Dense heads stream 2% slower this way than with
// a split's pieces adjacent in the grid; the GQA batch as a whole is 1%
// faster, and 7% faster over 8-bit pages.
__device__ __forceinline__ Item plan_item(const MicroParams& p, int x) {
  Item it;
  const int per_piece = p.n_items / p.chunks;
  it.c = x / per_piece;
  x -= it.c * per_piece;
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
  it.pa = it.pb = 0;
  if (it.t0 < it.t1) {
    it.pa = it.t0 / P;
    it.pb = (it.t1 + P - 1) / P;
  }
  return it;
}

// Sum of an int over the 64 lanes of a wave; every lane receives it.
__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// The kept pages of a piece: ordinals [o0, o1) among the split's kept pages.
struct Piece {
  int o0, o1;
};

// Cuts a split into pieces by its kept pages: the K kept pages of [pa, pb)
// (mask != 0; every page without a mask) form n = clamp(round(K / T), 1, C)
// runs of equal length, T = p.piece_pages, C = p.chunks, and piece c takes
// run c (nothing when c >= n).  A piece's fixed cost -- the chain of
// metadata loads before its first slab, the compaction, the end-of-item
// combine, its partial -- is the same whatever its length, so pieces of
// about T pages keep that cost small next to the streaming time; cutting the
// logical range instead gives a block-sparse head's splits pieces of a
// quarter of the dense heads' size (1 MiB against 4 MiB on the GQA batch),
// which streamed 13% slower.  Every thread calls it (barriers inside).
__device__ __forceinline__ Piece plan_piece(const MicroParams& p, const Item& it, int* s_cnt) {
  Piece pc{0, 0};
  if (it.pa >= it.pb) return pc;
  int K = it.pb - it.pa;
  if (it.mrow != nullptr) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int n = 0;
    for (int lp = it.pa + (int)threadIdx.x; lp < it.pb; lp += kMicroThreads) n += it.mrow[lp] != 0;
    n = wave_sum_int(n);
    if (lane == 0) s_cnt[wave] = n;
    __syncthreads();
    K = __builtin_amdgcn_readfirstlane(s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3]);
    __syncthreads();  // s_cnt is reused by the compaction
  }
  const int T = p.piece_pages;
  const int n = max(1, min((int)(((long long)K + T / 2) / T), p.chunks));
  if (it.c < n) {
    pc.o0 = (int)(((long long)K * it.c) / n);
    pc.o1 = (int)(((long long)K * (it.c + 1)) / n);
  }
  return pc;
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

// Item number of the k-th item of work queue q: queue q holds the splits j
// with j % kQueues == q, ordered (piece, request, split, KV head) with the KV
// head fastest, so that the workgroups of one XCD read the tiles of all KV
// heads of one page range close together in time (a page-major pool keeps
// a page's heads side by side).  Items are numbered as in plan_item.
__device__ __forceinline__ int queue_item(const MicroParams& p, int q, int nj, int k) {
  const int kvh = k % p.Hkv;
  int r = k / p.Hkv;
  const int jj = r % nj;
  r /= nj;
  const int s = r % p.S;
  const int c = r / p.S;
  return (c * p.S + s) * p.Hkv * p.max_splits + kvh * p.max_splits + q + kQueues * jj;
}

// Runs body(x) for every work item x this workgroup owns (kFused: the
// kernel instance with the fused merge): item blockIdx.x for a one-per-item
// launch, or, for a persistent launch, items claimed one at a time from the
// work queues of p.queue.  The dispatcher places workgroup b on XCD
// b % kQueues, so a workgroup drains queue b % kQueues first (its XCD's
// share: each XCD then serves the same splits of every KV head, as a
// one-per-item launch of those shapes does), then the other queues in turn.
// The next claim is issued before the current item is processed, so its
// latency is hidden.  body may use LDS and barriers; every lane calls it
// with the same x.
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
  const int home = (int)(blockIdx.x % kQueues);
  const int per_split_set = p.chunks * p.S * p.Hkv;  // items per split index
  int qi = 0, q = home;
  auto splits_of = [&](int qq) { return qq < p.max_splits ? (p.max_splits - 1 - qq) / kQueues + 1 : 0; };
  int nj = splits_of(q);
  if (tid == 0) *s_claim = atomicAdd(p.queue + q * kQueueStride, 1);
  __syncthreads();
  int k = __builtin_amdgcn_readfirstlane(*s_claim);
  for (;;) {
    // a drained queue (or a counter not reset to 0): the next queue
    while (k < 0 || k >= per_split_set * nj) {
      if (++qi == kQueues) return;
      q = (home + qi) % kQueues;
      nj = splits_of(q);
      __syncthreads();  // every lane has read s_claim
      if (tid == 0) *s_claim = atomicAdd(p.queue + q * kQueueStride, 1);
      __syncthreads();
      k = __builtin_amdgcn_readfirstlane(*s_claim);
    }
    int next = 0;
    if (tid == 0) next = atomicAdd(p.queue + q * kQueueStride, 1);
    body(queue_item(p, q, nj, k));
    __syncthreads();  // the item's LDS (page list, combine) is free again
    if (tid == 0) *s_claim = next;
    __syncthreads();
    k = __builtin_amdgcn_readfirstlane(*s_claim);
  }
}

// Compacts into LDS (physical and logical page ids, in logical order) the
// kept pages of ordinals [w0, w1) (w1 - w0 <= kPageCap) among the kept pages
// of the logical pages [lp, pb), with wave ballots over groups of 256 pages.
// (lp, ord) is the resume point: the group starting at logical page lp,
// whose first kept page has ordinal ord <= w0; it is left at the group that
// holds ordinal w1, where the next window starts.  The block-table entries
// of a group are loaded together with its mask bytes (the two loads are not
// chained; an entry of a masked page is read and not used).  Every thread
// must call it; returns the number of pages stored (w1 - w0 unless the
// split has fewer kept pages).
__device__ __forceinline__ int compact_window(int& lp, int& ord, int pb, int w0, int w1,
                                              const uint8_t* mrow, const int32_t* trow,
                                              int* s_phys, int* s_lp, int* s_cnt) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  int got = w0;  // ordinals below `got` (and >= w0) are stored
  while (lp < pb) {
    const int x = lp + tid;
    const bool in = x < pb;
    const int phys = in ? trow[x] : 0;
    const bool keep = in && (mrow == nullptr || mrow[x] != 0);
    const uint64_t bal = __ballot(keep);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = ord;
    for (int w = 0; w < wave; ++w) off += s_cnt[w];
    const int gend = __builtin_amdgcn_readfirstlane(ord + s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3]);
    const int o = off + pre;
    if (keep && o >= w0 && o < w1) {
      s_phys[o - w0] = phys;
      s_lp[o - w0] = x;
    }
    __syncthreads();  // s_cnt is rewritten by the next group
    if (gend > w1) {  // the group also holds pages of the next window: resume here
      got = w1;
      break;
    }
    got = max(got, gend);
    ord = gend;
    lp += kMicroThreads;
    if (ord == w1) break;
  }
  return got - w0;
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
//
// What the fused merge relies on.  On gfx942 and gfx950 the compiler lowers
// a monotonic agent-scope atomic store to a global_store with sc1 and a
// monotonic agent-scope atomic load to a global_load with sc1 (the AMDGPU
// backend's memory model for these targets): the store is made coherent
// across the XCDs when it completes, and the load does not hit a stale
// line in this XCD's L2.  A writer waits for its stores to complete
// (s_waitcnt vmcnt(0)) before the barrier that precedes its counter update,
// and the reader loads only after its own counter update returned the last
// count, so every partial it loads completed before it was issued.  Under
// the HIP/C++ memory model relaxed accesses to different locations are not
// ordered by this; the formal pair (a release counter update per item, an
// acquire fence in the last arrival) compiles to an L2 write-back per item
// and an L2 invalidate per group and measured 1.8x (C2: 355 vs 194 us) to
// 2.8x (C3: 2852 vs 1009 us) slower, so the kernels keep the lowering-based
// form, and the fused instances build only for the two targets whose
// lowering is this.
#if defined(__HIP_DEVICE_COMPILE__) && !defined(__gfx950__) && !defined(__gfx942__)
#error "the fused merge relies on the gfx942/gfx950 lowering of agent-scope atomics"
#endif
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
  // The partials were written as device-scope atomic stores and are read
  // back the same way; waiting until they have completed orders them before
  // the counter (the rule stated at store_dev).
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
// workgroup per resident slot, each claiming items one at a time from the
// per-XCD work queues (for_each_item).
template <class Kernel>
hipError_t launch_micro_kernel(Kernel kernel, int wg_per_cu, MicroParams p, hipStream_t stream);

// The step in one launch or two (p.group_count != null).  One launch: the
// kernel instance with the fused merge.  Two: the plain instance writes
// every piece's partial into p.MA / p.m / p.e (the workspace), then the merge
// kernel folds the max_splits * chunks partials of each (request, query
// head) -- the same aggregation rule, associative, so the pieces need no
// separate combine.  The fused merge saves a launch and the partials' round
// trip but makes every item count its group up, and the group's last item
// merge alone.  Measured with both forms timed in one process, it wins
// where the grid is one round of workgroups (C1: 20.8 against 24.4 us) and
// loses on long grids of short single-head items (C2: 193 against 170 us),
// on the persistent work queues (C3: 913 against 901 us) and on the
// grouped-query batch (C5: 1614 against 1584 us over bf16 pages, 876
// against 859 over 8-bit, 513 against 500 over 4-bit), where the merge's
// tail on the last item of each group outweighs the saved launch.
// fuse = 1 or 2 forces a form.
template <int D, class KPlain, class KFused>
hipError_t launch_micro_step(KPlain plain, KFused fused, int wg_per_cu, MicroParams p,
                             hipStream_t stream) {
  if (p.group_count == nullptr) return launch_micro_kernel(plain, wg_per_cu, p, stream);
  bool one = p.fuse == 1;
  if (p.fuse == 0) {
    const void* fn = reinterpret_cast<const void*>(plain);
    const int slots = resident_slots(fn, occupancy_lds(fn, wg_per_cu));
    one = p.n_items <= slots;
    // a fused instance that spills registers (the merge's code on top of the
    // largest slab loops: 4-bit pages with 64-token slabs, G = 8) runs its
    // slab loop through scratch memory; measured on the GQA batch over 4-bit
    // pages, 707 us forced to one launch against 670 us in two
    hipFuncAttributes fa;
    if (one && hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(fused)) == hipSuccess &&
        fa.localSizeBytes > 0)
      one = false;
  }
  if (one) return launch_micro_kernel(fused, wg_per_cu, p, stream);
  MicroParams q = p;
  q.group_count = nullptr;
  q.out = nullptr;
  const hipError_t err = launch_micro_kernel(plain, wg_per_cu, q, stream);
  if (err != hipSuccess) return err;
  return launch_merge(q.MA, q.m, q.e, p.out, p.S, p.Hq, D, p.max_splits * p.chunks, stream);
}

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
    } else {
      p.queue = nullptr;
    }
  }
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kMicroThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace da
