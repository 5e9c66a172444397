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

// One work item: (request s, KV head kvh, split j, chunk c).  The chunk is a
// contiguous range of the split's logical pages; its tokens are
// [t0, t1) = split range intersected with the chunk's pages.
struct Item {
  int s, kvh, j, c;
  int t0, t1;    // token range (empty if t0 >= t1)
  int lp0, lp1;  // logical page range to scan
};

__device__ __forceinline__ Item decode_item(const MicroParams& p) {
  Item it;
  int x = blockIdx.x;
  it.c = x % p.chunks;
  x /= p.chunks;
  it.j = x % p.max_splits;
  x /= p.max_splits;
  it.kvh = x % p.Hkv;
  it.s = x / p.Hkv;
  const int P = p.P;
  int Ls = p.lens[it.s];
  Ls = max(0, min(Ls, p.max_pages * P));
  const int32_t* sb = p.bounds + ((size_t)it.s * (p.bounds_per_head ? p.Hkv : 1) +
                                  (p.bounds_per_head ? it.kvh : 0)) *
                                     (size_t)(p.max_splits + 1);
  int t0 = max(sb[it.j], 0);
  int t1 = min(sb[it.j + 1], Ls);
  if (t0 < t1) {
    const int a = t0 / P, b = (t1 + P - 1) / P;  // split's pages
    const int n = b - a;
    const int ca = a + (int)(((long long)n * it.c) / p.chunks);
    const int cb = a + (int)(((long long)n * (it.c + 1)) / p.chunks);
    t0 = max(t0, ca * P);
    t1 = min(t1, cb * P);
  }
  it.t0 = t0;
  it.t1 = t1;
  it.lp0 = t0 < t1 ? t0 / P : 0;
  it.lp1 = t0 < t1 ? (t1 + P - 1) / P : 0;
  return it;
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
};

// Combines the four waves' triples and writes the item's partials.  Each
// wave supplies, per head g: raw-dot maximum wm[g] and exp-sum we[g] (valid
// in every lane) and, in the lanes of its first row (lane < LPT), the value
// sums acc[g][k] for dimensions lane*EPL + k.  Output index
// ((s*Hq + h)*max_splits + j)*chunks + c.
template <int G, int D, int LPT, int EPL>
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
    p.MA[o * D + d] = num;
    if (d == 0) {
      p.m[o] = M * p.scale;
      p.e[o] = den;
    }
  }
}

}  // namespace da
