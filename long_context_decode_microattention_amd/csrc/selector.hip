// Hierarchical page selection for retrieval heads (LServe blog page, section
// 2.2.2 "解码阶段创新" and section 3.1.2 "动态稀疏的层次化选择"): a physical
// page of P tokens is made of logical pages of `logical` tokens; every
// logical page keeps the per-dimension maximum and minimum of its keys; a
// physical page's importance for a query is the largest, over its logical
// pages, of the bound those statistics put on q . k; the top-K physical pages
// become the block mask the MicroAttention kernels consume.
//
// Three kernels:
//   page_stats_kernel   K pool -> statistics pool [NP, Hkv, P/logical, 2, D]
//                       (same element type as K; max/min of stored values are
//                       stored values, so bf16 statistics are exact).
//   page_scores_kernel  statistics + q -> score per (request, KV head, page).
//                       Per dimension the bound picks kmax where q_d >= 0 and
//                       kmin where q_d < 0 (one bit-select per element), then
//                       a dot product: sum_d max(q_d kmax_d, q_d kmin_d); the
//                       maximum over the group's query heads and over the
//                       valid logical pages of the physical page.
//   select_pages_kernel scores -> uint8 mask: forced first/last pages plus the
//                       `budget` best others, by a most-significant-digit-first
//                       radix select over order-preserving integer keys, equal
//                       keys going to the lower page index.
#include "device_common.h"
#include "launch.h"

namespace da {
namespace {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kScorePagesPerItem = 64;  // physical pages per score workgroup
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;

// Element layout of one D-wide row: each lane holds 16 bytes of it.
template <int DT, int D>
struct Row {
  static constexpr int ES = DT == 0 ? 4 : 2;  // element bytes
  static constexpr int RB = D * ES;           // row bytes
  static constexpr int LPR = RB / 16;         // lanes per row
  static constexpr int RPW = kWave / LPR;     // rows per wave load
  static constexpr int EPL = 16 / ES;         // elements per lane
};

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint32_t word(const uint4& w, int i) {
  return i == 0 ? w.x : (i == 1 ? w.y : (i == 2 ? w.z : w.w));
}

// 16 bytes of DT elements -> EPL floats (exact).
template <int DT>
__device__ __forceinline__ void unpack(const uint4& w, float (&x)[Row<DT, 64>::EPL]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = word(w, i);
    if constexpr (DT == 0) {
      x[i] = __builtin_bit_cast(float, u);
    } else {
      x[2 * i] = bf16_lo(u);
      x[2 * i + 1] = bf16_hi(u);
    }
  }
}

// EPL floats that are exactly representable in DT -> 16 bytes.
template <int DT>
__device__ __forceinline__ uint4 pack(const float (&x)[Row<DT, 64>::EPL]) {
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == 0) {
      u[i] = __builtin_bit_cast(uint32_t, x[i]);
    } else {
      u[i] = (__builtin_bit_cast(uint32_t, x[2 * i]) >> 16) |
             (__builtin_bit_cast(uint32_t, x[2 * i + 1]) & 0xFFFF0000u);
    }
  }
  return make_uint4(u[0], u[1], u[2], u[3]);
}

__device__ __forceinline__ int clamp_len(const int32_t* lens, int s, int max_tokens) {
  return max(0, min(lens[s], max_tokens));
}

// ---------------------------------------------------------------------------
// statistics
// ---------------------------------------------------------------------------

// One workgroup per (request, logical page index) of the table; its waves
// take the (KV head, logical sub-page) pairs of the physical page in turn.
// A wave folds the sub-page's valid rows per lane (RPW rows per load), then
// across the rows of the wave; row 0 stores kmax, row 1 kmin.
template <int DT, int D>
__global__ __launch_bounds__(kSelThreads) void page_stats_kernel(SelectorParams p) {
  using R = Row<DT, D>;
  const int s = blockIdx.x / p.max_pages;
  const int lp = blockIdx.x - s * p.max_pages;
  const int L = clamp_len(p.lens, s, p.max_pages * p.P);
  if (lp * p.P >= L) return;
  const long long phys = p.table[(size_t)s * p.max_pages + lp];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int row = lane / R::LPR;
  const int col = lane - row * R::LPR;
  const int NL = p.P / p.logical;
  const int tasks = p.Hkv * NL;
  for (int t = wave; t < tasks; t += kSelWaves) {
    const int kvh = t / NL;
    const int sub = t - kvh * NL;
    const int slot0 = sub * p.logical;
    const char* base = static_cast<const char*>(p.k) +
                       ((size_t)phys * p.Hkv + kvh) * p.P * R::RB + (size_t)col * 16;
    float hi[R::EPL], lo[R::EPL];
#pragma unroll
    for (int i = 0; i < R::EPL; ++i) {
      hi[i] = neg_inf();
      lo[i] = -neg_inf();
    }
    for (int r = row; r < p.logical; r += R::RPW) {
      const int slot = slot0 + r;
      if (lp * p.P + slot < L) {
        float x[R::EPL];
        unpack<DT>(load_stream16(base + (size_t)slot * R::RB), x);
#pragma unroll
        for (int i = 0; i < R::EPL; ++i) {
          hi[i] = fmaxf(hi[i], x[i]);
          lo[i] = fminf(lo[i], x[i]);
        }
      }
    }
#pragma unroll
    for (int off = R::LPR; off < kWave; off <<= 1) {
#pragma unroll
      for (int i = 0; i < R::EPL; ++i) {
        hi[i] = fmaxf(hi[i], __shfl_xor(hi[i], off, kWave));
        lo[i] = fminf(lo[i], __shfl_xor(lo[i], off, kWave));
      }
    }
    if (row < 2) {
      const bool any = lp * p.P + slot0 < L;
      float v[R::EPL];
#pragma unroll
      for (int i = 0; i < R::EPL; ++i) v[i] = any ? (row == 0 ? hi[i] : lo[i]) : 0.f;
      char* out = static_cast<char*>(p.stats) +
                  ((((size_t)phys * p.Hkv + kvh) * NL + sub) * 2 + row) * R::RB + (size_t)col * 16;
      *reinterpret_cast<uint4*>(out) = pack<DT>(v);
    }
  }
}

// ---------------------------------------------------------------------------
// scores
// ---------------------------------------------------------------------------

// Sign masks of q: all ones over an element where q_d >= 0 (that element of
// the bound uses kmax), zero where q_d < 0 (it uses kmin).
template <int DT>
__device__ __forceinline__ uint4 sign_select(const uint4& q) {
  uint32_t m[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = word(q, i);
    if constexpr (DT == 0) {
      m[i] = (u & 0x80000000u) ? 0u : 0xFFFFFFFFu;
    } else {
      m[i] = ((u & 0x8000u) ? 0u : 0x0000FFFFu) | ((u & 0x80000000u) ? 0u : 0xFFFF0000u);
    }
  }
  return make_uint4(m[0], m[1], m[2], m[3]);
}

// This lane's part of sum_d max(q_d kmax_d, q_d kmin_d).
template <int DT>
__device__ __forceinline__ float bound_part(const uint4& kmax, const uint4& kmin, const uint4& q,
                                            const uint4& msk) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t m = word(msk, i);
    const uint32_t sel = (word(kmax, i) & m) | (word(kmin, i) & ~m);
    if constexpr (DT == 0)
      acc = fmaf(__builtin_bit_cast(float, word(q, i)), __builtin_bit_cast(float, sel), acc);
    else
      acc = dot2_bf16(sel, word(q, i), acc);
  }
  return acc;
}

// One workgroup per (request, KV head, run of kScorePagesPerItem pages).  A
// wave step covers RPW logical pages (one per row of LPR lanes): PPS whole
// physical pages when a physical page has fewer logical pages than a wave
// has rows, else one physical page over SPP steps.
template <int DT, int D, int G>
__global__ __launch_bounds__(kSelThreads) void page_scores_kernel(SelectorParams p) {
  using R = Row<DT, D>;
  const int runs = (p.max_pages + kScorePagesPerItem - 1) / kScorePagesPerItem;
  int x = blockIdx.x;
  const int run = x % runs;
  x /= runs;
  const int kvh = x % p.Hkv;
  const int s = x / p.Hkv;
  const int lp0 = run * kScorePagesPerItem;
  const int lp1 = min(lp0 + kScorePagesPerItem, p.max_pages);
  float* out = p.scores + ((size_t)s * p.Hkv + kvh) * p.max_pages;
  const int tid = threadIdx.x;
  if (p.select != nullptr && p.select[kvh] == 0) {
    for (int lp = lp0 + tid; lp < lp1; lp += kSelThreads) out[lp] = neg_inf();
    return;
  }
  const int L = clamp_len(p.lens, s, p.max_pages * p.P);
  const int npg = (L + p.P - 1) / p.P;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int row = lane / R::LPR;
  const int col = lane - row * R::LPR;

  uint4 qv[G], qm[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    qv[g] = load16(static_cast<const char*>(p.q) +
                   ((size_t)s * p.Hq + (size_t)kvh * G + g) * R::RB + (size_t)col * 16);
    qm[g] = sign_select<DT>(qv[g]);
  }

  const int NL = p.P / p.logical;
  const int rows_per_page = min(NL, R::RPW);  // rows of one page within a step
  const int PPS = R::RPW / rows_per_page;     // physical pages per step
  const int SPP = NL / rows_per_page;         // steps per physical page
  const int rowpage = row / rows_per_page;
  const int rowsub = row - rowpage * rows_per_page;
  const size_t head_stride = (size_t)NL * 2 * R::RB;  // one (page, KV head) of statistics

  for (int pg = lp0 + wave * PPS; pg < lp1; pg += kSelWaves * PPS) {
    const int lp = pg + rowpage;
    const bool pvalid = lp < lp1 && lp < npg;
    const long long phys = pvalid ? p.table[(size_t)s * p.max_pages + lp] : 0;
    const char* st = static_cast<const char*>(p.stats) + ((size_t)phys * p.Hkv + kvh) * head_stride +
                     (size_t)col * 16;
    float best = neg_inf();
    for (int step = 0; step < SPP; ++step) {
      const int sub = rowsub + step * rows_per_page;
      const bool valid = pvalid && lp * p.P + sub * p.logical < L;
      uint4 kmax = make_uint4(0, 0, 0, 0), kmin = make_uint4(0, 0, 0, 0);
      if (valid) {
        kmax = load16(st + (size_t)sub * 2 * R::RB);
        kmin = load16(st + (size_t)sub * 2 * R::RB + R::RB);
      }
      float h = neg_inf();
#pragma unroll
      for (int g = 0; g < G; ++g) h = fmaxf(h, group_sum<R::LPR>(bound_part<DT>(kmax, kmin, qv[g], qm[g])));
      if (valid) best = fmaxf(best, h);
    }
    for (int off = R::LPR; off < R::LPR * rows_per_page; off <<= 1)
      best = fmaxf(best, __shfl_xor(best, off, kWave));
    if (col == 0 && rowsub == 0 && lp < lp1) out[lp] = best;
  }
}

// ---------------------------------------------------------------------------
// top-K
// ---------------------------------------------------------------------------

// Unsigned key with the order of the float (negative zero taken as zero).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One workgroup per (request, KV head).
__global__ __launch_bounds__(kTopkThreads) void select_pages_kernel(SelectorParams p) {
  __shared__ int s_hist[256];
  __shared__ int s_need, s_digit;
  __shared__ int s_wcnt[kTopkWaves];
  const int s = blockIdx.x / p.Hkv;
  const int kvh = blockIdx.x - s * p.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int L = clamp_len(p.lens, s, p.max_pages * p.P);
  const int npg = (L + p.P - 1) / p.P;
  const float* sc = p.scores + ((size_t)s * p.Hkv + kvh) * p.max_pages;
  uint8_t* mrow = p.mask + ((size_t)s * p.Hkv + kvh) * p.max_pages;

  const bool selected = p.select == nullptr || p.select[kvh] != 0;
  const int lo = selected ? min(p.keep_first, npg) : npg;
  const int hi = selected ? max(npg - p.keep_last, lo) : npg;
  // pages outside [lo, hi) are forced (below npg) or zero (at or beyond npg)
  for (int i = tid; i < p.max_pages; i += kTopkThreads)
    if (i < lo || i >= hi) mrow[i] = i < npg ? 1 : 0;
  const int n = hi - lo;
  if (n <= 0) return;
  if (p.budget >= n || p.budget <= 0) {
    const uint8_t v = p.budget > 0 ? 1 : 0;
    for (int i = lo + tid; i < hi; i += kTopkThreads) mrow[i] = v;
    return;
  }

  // the budget-th largest key, one 8-bit digit at a time from the top
  uint32_t prefix = 0, pmask = 0;
  int need = p.budget;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kTopkThreads) s_hist[i] = 0;
    __syncthreads();
    for (int i = lo + tid; i < hi; i += kTopkThreads) {
      const uint32_t k = order_key(sc[i]);
      if ((k & pmask) == prefix) atomicAdd(&s_hist[(k >> shift) & 0xFFu], 1);
    }
    __syncthreads();
    if (tid == 0) {
      // keys matching the prefix number at least `need`, so the scan stops
      int cum = 0, d = 255;
      while (d > 0 && cum + s_hist[d] < need) cum += s_hist[d--];
      s_need = need - cum;
      s_digit = d;
    }
    __syncthreads();
    need = s_need;
    prefix |= (uint32_t)s_digit << shift;
    pmask |= 0xFFu << shift;
    __syncthreads();  // s_hist is cleared again by the next digit
  }

  // keep keys above the threshold and the first `need` equal ones
  int base = 0;
  for (int c0 = lo; c0 < hi; c0 += kTopkThreads) {
    const int i = c0 + tid;
    const bool in = i < hi;
    const uint32_t k = in ? order_key(sc[i]) : 0u;
    const bool eq = in && k == prefix;
    const uint64_t bal = __ballot(eq);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_wcnt[wave] = __popcll(bal);
    __syncthreads();
    int off = base, tot = 0;
    for (int w = 0; w < kTopkWaves; ++w) {
      if (w < wave) off += s_wcnt[w];
      tot += s_wcnt[w];
    }
    if (in) mrow[i] = (k > prefix || (eq && off + pre < need)) ? 1 : 0;
    base += tot;
    __syncthreads();
  }
}

template <int DT, int D>
hipError_t scores_g(int G, const SelectorParams& p, dim3 grid, hipStream_t stream) {
  switch (G) {
    case 1: hipLaunchKernelGGL((page_scores_kernel<DT, D, 1>), grid, dim3(kSelThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((page_scores_kernel<DT, D, 2>), grid, dim3(kSelThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((page_scores_kernel<DT, D, 4>), grid, dim3(kSelThreads), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((page_scores_kernel<DT, D, 8>), grid, dim3(kSelThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool selector_supported(int dtype, int D, int G, int P, int logical) {
  if (dtype != 0 && dtype != 1) return false;
  if (D != 64 && D != 128) return false;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  if (logical != 8 && logical != 16 && logical != 32 && logical != 64) return false;
  return P >= logical && P % logical == 0 && ((P / logical) & (P / logical - 1)) == 0;
}

hipError_t launch_page_stats(const SelectorParams& p, int dtype, int D, hipStream_t stream) {
  const long long grid = (long long)p.S * p.max_pages;
  if (grid < 1) return hipSuccess;
  const dim3 g((unsigned)grid), b(kSelThreads);
  if (dtype == 0 && D == 64) hipLaunchKernelGGL((page_stats_kernel<0, 64>), g, b, 0, stream, p);
  else if (dtype == 0 && D == 128) hipLaunchKernelGGL((page_stats_kernel<0, 128>), g, b, 0, stream, p);
  else if (dtype == 1 && D == 64) hipLaunchKernelGGL((page_stats_kernel<1, 64>), g, b, 0, stream, p);
  else if (dtype == 1 && D == 128) hipLaunchKernelGGL((page_stats_kernel<1, 128>), g, b, 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_page_scores(const SelectorParams& p, int dtype, int D, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  const long long runs = (p.max_pages + kScorePagesPerItem - 1) / kScorePagesPerItem;
  const long long grid = (long long)p.S * p.Hkv * runs;
  if (grid < 1) return hipSuccess;
  const dim3 g((unsigned)grid);
  if (dtype == 0) return D == 64 ? scores_g<0, 64>(G, p, g, stream) : scores_g<0, 128>(G, p, g, stream);
  return D == 64 ? scores_g<1, 64>(G, p, g, stream) : scores_g<1, 128>(G, p, g, stream);
}

hipError_t launch_select_pages(const SelectorParams& p, hipStream_t stream) {
  const long long grid = (long long)p.S * p.Hkv;
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(select_pages_kernel, dim3((unsigned)grid), dim3(kTopkThreads), 0, stream, p);
  return hipGetLastError();
}

long long score_launch_items(int S, int Hkv, int max_pages) {
  return (long long)S * Hkv * ((max_pages + kScorePagesPerItem - 1) / kScorePagesPerItem);
}

}  // namespace da
