// Hierarchical page selection for retrieval heads (LServe blog page, section
// 2.2.2 "解码阶段创新" and section 3.1.2 "动态稀疏的层次化选择"): a physical
// page of P tokens is made of logical pages of `logical` tokens; every
// logical page keeps the per-dimension maximum and minimum of its keys; a
// physical page's importance for a query is the largest, over its logical
// pages, of the bound those statistics put on q . k; the top-K physical pages
// become the block mask the MicroAttention kernels consume.
//
// Three kernels, all streaming (HBM-bound or latency-bound, no dense
// contraction):
//   page_stats_kernel   K pool -> statistics pool [Hkv, NP, P/logical, 2, D]
//                       (same element type as K; max/min of stored values are
//                       stored values, so bf16 statistics are exact).  A lane
//                       owns 16 bytes of one (KV head, logical page) column
//                       and folds every row of it, 16 rows in flight, so no
//                       cross-lane reduction is needed; the statistics go out
//                       with non-temporal stores (plain stores, mixed into
//                       the read stream, cost 10% more time).  They are
//                       head-major: one KV head's pages form one contiguous
//                       run, which is what the score kernel streams (measured
//                       6.5 TB/s against 5.5 TB/s for page-major blocks of
//                       2 KiB at a 16 KiB stride, on the 512K GQA shape).
//   page_scores_kernel  statistics + q -> score per (request, KV head, page).
//                       Per dimension the bound picks kmax where q_d >= 0 and
//                       kmin where q_d < 0 (one bit-select per element), then
//                       a dot product: sum_d max(q_d kmax_d, q_d kmin_d); the
//                       maximum over the group's query heads, then (through
//                       LDS) over the valid logical pages of a physical page.
//   select_pages_kernel scores -> uint8 mask: forced first/last pages plus the
//                       `budget` best others.  Keys (order-preserving integer
//                       images of the scores) stay in registers; the K-th
//                       largest key is found one bit at a time from the top
//                       by counting keys at or above a candidate (ballots,
//                       one barrier per bit); equal keys go to the lower page
//                       index through one block-wide prefix count.
#include "device_common.h"
#include "launch.h"

namespace da {
namespace {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kStatsUnroll = 16;           // rows of one column in flight per lane
constexpr int kScoreLogicalPerItem = 256;  // logical pages per score workgroup
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kTopkMaxKeys = 64;           // keys per thread: up to 65536 candidates

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

__device__ __forceinline__ bool head_selected(const uint8_t* select, int kvh) {
  return select == nullptr || select[kvh] != 0;
}

// ---------------------------------------------------------------------------
// statistics
// ---------------------------------------------------------------------------

// One workgroup per (request, logical page index) of the table.  The page's
// (KV head, logical sub-page) columns are numbered t = kvh * NL + sub, which
// is also their order in the pool: column t starts t * logical rows into the
// physical page.  A wave job covers TPW consecutive columns (one 16-byte
// slice per lane), so each of its loads reads TPW contiguous row segments;
// its statistics go to row pair sub of page phys in head kvh's run.
template <int DT, int D>
__global__ __launch_bounds__(kSelThreads) void page_stats_kernel(SelectorParams p) {
  using R = Row<DT, D>;
  constexpr int TPW = kWave / R::LPR;
  const int s = blockIdx.x / p.max_pages;
  const int lp = blockIdx.x - s * p.max_pages;
  const int L = clamp_len(p.lens, s, p.max_pages * p.P);
  if (lp * p.P >= L) return;
  const long long phys = p.table[(size_t)s * p.max_pages + lp];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int tsk = lane / R::LPR;
  const int col = lane - tsk * R::LPR;
  const int NL = p.P / p.logical;
  const int tasks = p.Hkv * NL;
  // the (page, KV head) tile: [phys][kvh] of a page-major pool or [kvh][phys]
  // of a head-major one; column t = kvh * NL + sub starts sub * logical rows in
  const char* kpool = static_cast<const char*>(p.k) + (size_t)col * 16;
  const size_t tile = (size_t)p.P * R::RB;
  const size_t head_stride = (size_t)p.NP * NL * 2 * R::RB;
  char* spage = static_cast<char*>(p.stats) + (size_t)phys * NL * 2 * R::RB + (size_t)col * 16;

  for (int t0 = wave * TPW; t0 < tasks; t0 += kSelWaves * TPW) {
    const int t = t0 + tsk;
    bool write = false;
    int nv = 0;  // rows of this column below L
    int kvh = 0, sub = 0;
    if (t < tasks) {
      kvh = t / NL;
      sub = t - kvh * NL;
      write = head_selected(p.select, kvh);
      if (write) nv = max(0, min(p.logical, L - (lp * p.P + sub * p.logical)));
    }
    const size_t tile_id = p.head_major ? (size_t)kvh * p.NP + phys : (size_t)phys * p.Hkv + kvh;
    const char* src = kpool + tile_id * tile + (size_t)sub * p.logical * R::RB;
    float hi[R::EPL], lo[R::EPL];
#pragma unroll
    for (int i = 0; i < R::EPL; ++i) {
      hi[i] = neg_inf();
      lo[i] = -neg_inf();
    }
    for (int r0 = 0; r0 < nv; r0 += kStatsUnroll) {
      uint4 w[kStatsUnroll];
#pragma unroll
      for (int u = 0; u < kStatsUnroll; ++u)
        w[u] = r0 + u < nv ? load_stream16(src + (size_t)(r0 + u) * R::RB) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < kStatsUnroll; ++u) {
        if (r0 + u < nv) {
          float x[R::EPL];
          unpack<DT>(w[u], x);
#pragma unroll
          for (int i = 0; i < R::EPL; ++i) {
            hi[i] = fmaxf(hi[i], x[i]);
            lo[i] = fminf(lo[i], x[i]);
          }
        }
      }
    }
    if (write) {
      if (nv == 0) {
#pragma unroll
        for (int i = 0; i < R::EPL; ++i) hi[i] = lo[i] = 0.f;
      }
      char* dst = spage + (size_t)kvh * head_stride + (size_t)sub * 2 * R::RB;
      store_stream16(dst, pack<DT>(hi));
      store_stream16(dst + R::RB, pack<DT>(lo));
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

// Physical pages per score workgroup for NL logical pages per physical page.
__host__ __device__ __forceinline__ int score_pages_per_item(int NL) {
  return kScoreLogicalPerItem / NL;
}

// One workgroup per (request, KV head, run of kScoreLogicalPerItem logical
// pages).  The run's block-table entries are staged in LDS first; each wave
// load then covers RPW logical pages (one per row of LPR lanes), U loads of
// kmax and kmin in flight per lane (4 measured faster than 8 or 16: more
// waves stay resident); the per-logical-page bounds go to LDS and are folded
// per physical page at the end.
template <int DT, int D, int G>
__global__ __launch_bounds__(kSelThreads) void page_scores_kernel(SelectorParams p) {
  using R = Row<DT, D>;
  constexpr int U = 4;
  __shared__ int s_phys[kScoreLogicalPerItem];
  __shared__ float s_bound[kScoreLogicalPerItem];
  const int NL = p.P / p.logical;
  const int nl_shift = __builtin_ctz(NL);
  const int ppi = score_pages_per_item(NL);
  const int runs = (p.max_pages + ppi - 1) / ppi;
  int x = blockIdx.x;
  const int run = x % runs;
  x /= runs;
  const int kvh = x % p.Hkv;
  const int s = x / p.Hkv;
  const int lp0 = run * ppi;
  const int lp1 = min(lp0 + ppi, p.max_pages);
  float* out = p.scores + ((size_t)s * p.Hkv + kvh) * p.max_pages;
  const int tid = threadIdx.x;
  const int L = clamp_len(p.lens, s, p.max_pages * p.P);
  const int lpv = min(lp1, (L + p.P - 1) / p.P);  // end of the run's pages below L
  if (!head_selected(p.select, kvh) || lpv <= lp0) {
    for (int lp = lp0 + tid; lp < lp1; lp += kSelThreads) out[lp] = neg_inf();
    return;
  }
  for (int i = tid; i < lpv - lp0; i += kSelThreads)
    s_phys[i] = p.table[(size_t)s * p.max_pages + lp0 + i];

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
  __syncthreads();

  const int nlog = (lpv - lp0) << nl_shift;
  const size_t page_stride = (size_t)NL * 2 * R::RB;
  const char* st = static_cast<const char*>(p.stats) + (size_t)kvh * p.NP * page_stride + (size_t)col * 16;
  for (int base = wave * R::RPW * U; base < nlog; base += kSelWaves * R::RPW * U) {
    uint4 kmax[U], kmin[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int li = base + u * R::RPW + row;
      const int pl = li >> nl_shift;
      const int sub = li & (NL - 1);
      valid[u] = li < nlog && (lp0 + pl) * p.P + sub * p.logical < L;
      kmax[u] = kmin[u] = make_uint4(0, 0, 0, 0);
      if (valid[u]) {
        const char* src = st + (size_t)s_phys[pl] * page_stride + (size_t)sub * 2 * R::RB;
        kmax[u] = load_stream16(src);
        kmin[u] = load_stream16(src + R::RB);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float h = neg_inf();
#pragma unroll
      for (int g = 0; g < G; ++g)
        h = fmaxf(h, group_sum<R::LPR>(bound_part<DT>(kmax[u], kmin[u], qv[g], qm[g])));
      const int li = base + u * R::RPW + row;
      if (col == 0 && li < nlog) s_bound[li] = valid[u] ? h : neg_inf();
    }
  }
  __syncthreads();
  for (int i = tid; i < lp1 - lp0; i += kSelThreads) {
    float best = neg_inf();
    if (lp0 + i < lpv)
      for (int sub = 0; sub < NL; ++sub) best = fmaxf(best, s_bound[(i << nl_shift) + sub]);
    out[lp0 + i] = best;
  }
}

// ---------------------------------------------------------------------------
// top-K
// ---------------------------------------------------------------------------

// Unsigned key with the order of the float (negative zero taken as zero).
// Every non-NaN float maps above 0, which therefore marks an empty slot.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of keys >= c (gt = false) or > c (gt = true) over the wave.
template <int KPT>
__device__ __forceinline__ int wave_count(const uint32_t (&key)[KPT], uint32_t c, bool gt) {
  int n = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) n += __popcll(__ballot(gt ? key[j] > c : key[j] >= c));
  return n;
}

// One workgroup per (request, KV head).  Thread t owns candidates
// lo + t*KPT ... lo + t*KPT + KPT - 1, so thread order is page order.
template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void select_pages_kernel(SelectorParams p) {
  __shared__ int s_cnt[2][kTopkWaves];
  __shared__ int s_eq[kTopkWaves];
  __shared__ int s_gt[kTopkWaves];
  const int s = blockIdx.x / p.Hkv;
  const int kvh = blockIdx.x - s * p.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int L = clamp_len(p.lens, s, p.max_pages * p.P);
  const int npg = (L + p.P - 1) / p.P;
  const float* sc = p.scores + ((size_t)s * p.Hkv + kvh) * p.max_pages;
  uint8_t* mrow = p.mask + ((size_t)s * p.Hkv + kvh) * p.max_pages;

  const bool selected = head_selected(p.select, kvh);
  const int lo = selected ? min(p.keep_first, npg) : npg;
  const int hi = selected ? max(npg - p.keep_last, lo) : npg;
  // pages the next `horizon` appended tokens open stay kept while the
  // selection is reused
  const int npg_h = (int)min((long long)p.max_pages,
                             ((long long)L + p.horizon + p.P - 1) / p.P);
  // pages outside [lo, hi) are forced (below npg_h) or zero (at or beyond it)
  for (int i = tid; i < p.max_pages; i += kTopkThreads)
    if (i < lo || i >= hi) mrow[i] = i < npg_h ? 1 : 0;
  const int n = hi - lo;
  if (n <= 0) return;
  if (p.budget >= n || p.budget <= 0) {
    const uint8_t v = p.budget > 0 ? 1 : 0;
    for (int i = lo + tid; i < hi; i += kTopkThreads) mrow[i] = v;
    return;
  }

  const int first = lo + tid * KPT;
  uint32_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) key[j] = first + j < hi ? order_key(sc[first + j]) : 0u;

  // the largest T with #{key >= T} >= budget, i.e. the budget-th largest key
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    const int c = wave_count<KPT>(key, cand, false);
    if (lane == 0) s_cnt[bit & 1][wave] = c;
    __syncthreads();  // s_cnt[bit & 1] is written again two bits later, after the next barrier
    int tot = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) tot += s_cnt[bit & 1][w];
    if (tot >= p.budget) T = cand;
  }

  // keys above T are kept; of the keys equal to T the first `need` in page order
  int eq = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) eq += key[j] == T ? 1 : 0;
  int incl = eq;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  const int gt = wave_count<KPT>(key, T, true);
  if (lane == kWave - 1) s_eq[wave] = incl;
  if (lane == 0) s_gt[wave] = gt;
  __syncthreads();
  int before = incl - eq, total_gt = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    if (w < wave) before += s_eq[w];
    total_gt += s_gt[w];
  }
  const int need = p.budget - total_gt;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (first + j < hi) {
      bool keep = key[j] > T;
      if (key[j] == T) keep = before++ < need;
      mrow[first + j] = keep ? 1 : 0;
    }
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
  if (P < logical || P % logical != 0) return false;
  const int NL = P / logical;
  return (NL & (NL - 1)) == 0 && NL <= kScoreLogicalPerItem;
}

int select_max_pages() { return kTopkThreads * kTopkMaxKeys; }

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

long long score_launch_items(int S, int Hkv, int max_pages, int P, int logical) {
  const int ppi = score_pages_per_item(P / logical);
  return (long long)S * Hkv * ((max_pages + ppi - 1) / ppi);
}

hipError_t launch_page_scores(const SelectorParams& p, int dtype, int D, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  const long long grid = score_launch_items(p.S, p.Hkv, p.max_pages, p.P, p.logical);
  if (grid < 1) return hipSuccess;
  const dim3 g((unsigned)grid);
  if (dtype == 0) return D == 64 ? scores_g<0, 64>(G, p, g, stream) : scores_g<0, 128>(G, p, g, stream);
  return D == 64 ? scores_g<1, 64>(G, p, g, stream) : scores_g<1, 128>(G, p, g, stream);
}

hipError_t launch_select_pages(const SelectorParams& p, hipStream_t stream) {
  const long long grid = (long long)p.S * p.Hkv;
  if (grid < 1) return hipSuccess;
  const dim3 g((unsigned)grid), b(kTopkThreads);
  const int need = (p.max_pages + kTopkThreads - 1) / kTopkThreads;  // keys per thread
  if (need <= 1) hipLaunchKernelGGL(select_pages_kernel<1>, g, b, 0, stream, p);
  else if (need <= 2) hipLaunchKernelGGL(select_pages_kernel<2>, g, b, 0, stream, p);
  else if (need <= 4) hipLaunchKernelGGL(select_pages_kernel<4>, g, b, 0, stream, p);
  else if (need <= 8) hipLaunchKernelGGL(select_pages_kernel<8>, g, b, 0, stream, p);
  // each bit round counts every key a lane holds: steps of 4 past 8 keep the
  // count close to what the row needs (a 8193-page row takes 12, not 16)
  else if (need <= 12) hipLaunchKernelGGL(select_pages_kernel<12>, g, b, 0, stream, p);
  else if (need <= 16) hipLaunchKernelGGL(select_pages_kernel<16>, g, b, 0, stream, p);
  else if (need <= 24) hipLaunchKernelGGL(select_pages_kernel<24>, g, b, 0, stream, p);
  else if (need <= 32) hipLaunchKernelGGL(select_pages_kernel<32>, g, b, 0, stream, p);
  else if (need <= 48) hipLaunchKernelGGL(select_pages_kernel<48>, g, b, 0, stream, p);
  else if (need <= kTopkMaxKeys) hipLaunchKernelGGL(select_pages_kernel<kTopkMaxKeys>, g, b, 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace da
