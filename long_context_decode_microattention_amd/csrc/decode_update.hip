// Decode-time cache update and work planning for a reused page selection.
//
// append_kv_kernel     writes the new token's K and V rows of every (request,
//                      KV head) at logical position L_s through the block
//                      table, and keeps the logical-page key statistics
//                      current at write time (LServe blog page, section 3.1.2:
//                      the statistics are computed when the KV cache is
//                      written, adding no decode latency): the first token of
//                      a logical page sets kmax = kmin = k, later tokens fold
//                      into them with max / min (exact: stored values).
// append_kv_fp8_kernel the same write for 8-bit pages: the new rows are
//                      quantized (one scale per row, fp8_rows.h) and their
//                      codes and scales stored at the token's slot.
// split_bounds_kernel  split bounds over a head's kept pages (b splits, split
//                      j starting at the kept page of ordinal floor(j K / b)),
//                      computed on the device from the mask so a selection
//                      reused across a chunk of decode steps (LServe blog
//                      page, section 2.2.2, reusable page selector) never
//                      waits on the host.
//
// All three are tiny next to the attention step (one row per head, one mask
// row per head); they are written for latency: one wave per (request, KV
// head) for the appends, one workgroup per mask row for the bounds.
#include "fp8_rows.h"
#include "launch.h"

namespace da {
namespace {

constexpr int kAppendWaves = 4;
constexpr int kBoundsThreads = 256;
constexpr int kBoundsWaves = kBoundsThreads / kWave;
constexpr int kBoundsBits = 64;  // pages per thread held as a bit word

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Element-wise max (take_max) or min of two 16-byte groups of DT elements.
template <int DT>
__device__ __forceinline__ uint32_t fold_word(uint32_t a, uint32_t b, bool take_max) {
  if constexpr (DT == 0) {
    const float x = __builtin_bit_cast(float, a), y = __builtin_bit_cast(float, b);
    return __builtin_bit_cast(uint32_t, take_max ? fmaxf(x, y) : fminf(x, y));
  } else {
    const float xl = bf16_lo(a), yl = bf16_lo(b), xh = bf16_hi(a), yh = bf16_hi(b);
    const float l = take_max ? fmaxf(xl, yl) : fminf(xl, yl);
    const float h = take_max ? fmaxf(xh, yh) : fminf(xh, yh);
    return (__builtin_bit_cast(uint32_t, l) >> 16) | (__builtin_bit_cast(uint32_t, h) & 0xFFFF0000u);
  }
}

template <int DT>
__device__ __forceinline__ uint4 fold16(const uint4& a, const uint4& b, bool take_max) {
  return make_uint4(fold_word<DT>(a.x, b.x, take_max), fold_word<DT>(a.y, b.y, take_max),
                    fold_word<DT>(a.z, b.z, take_max), fold_word<DT>(a.w, b.w, take_max));
}

// One wave per (request, KV head).  The wave's lanes cover four 16-byte
// column groups of D-wide rows: part 0 = the K row, 1 = the V row, 2 = kmax,
// 3 = kmin of the logical page that receives the token (parts 2-3 only when
// statistics are kept for this head).
template <int DT, int D>
__global__ __launch_bounds__(kAppendWaves * kWave) void append_kv_kernel(AppendParams p) {
  constexpr int RB = D * (DT == 0 ? 4 : 2);
  constexpr int LPR = RB / 16;
  const int item = blockIdx.x * kAppendWaves + threadIdx.x / kWave;
  if (item >= p.S * p.Hkv) return;
  const int s = item / p.Hkv;
  const int kvh = item - s * p.Hkv;
  const int t = p.lens[s];
  if (t < 0 || t >= p.max_pages * p.P) return;  // full cache: nothing is written
  const int lp = t / p.P;
  const int slot = t - lp * p.P;
  const long long phys = p.table[(size_t)s * p.max_pages + lp];
  // the entry of the page that receives the token lies outside the range
  // da_check_inputs validates when L_s is a multiple of P: an entry outside
  // the pool writes nothing (wave-uniform)
  if (phys < 0 || phys >= p.NP) return;
  const bool stats = p.stats != nullptr && (p.select == nullptr || p.select[kvh] != 0);
  const int parts = stats ? 4 : 2;
  const size_t new_off = ((size_t)s * p.Hkv + kvh) * RB;
  const size_t tile_id = p.head_major ? (size_t)kvh * p.NP + phys : (size_t)phys * p.Hkv + kvh;
  const size_t row_off = (tile_id * p.P + slot) * RB;
  for (int c = threadIdx.x % kWave; c < parts * LPR; c += kWave) {
    const int part = c / LPR;
    const size_t col = (size_t)(c - part * LPR) * 16;
    if (part < 2) {
      const char* src = static_cast<const char*>(part == 0 ? p.k_new : p.v_new) + new_off + col;
      char* dst = static_cast<char*>(part == 0 ? p.k : p.v) + row_off + col;
      st16(dst, ld16(src));
    } else {
      const uint4 k = ld16(static_cast<const char*>(p.k_new) + new_off + col);
      const int NL = p.P / p.logical;
      const int sub = slot / p.logical;
      char* dst = static_cast<char*>(p.stats) +
                  ((((size_t)kvh * p.NP + phys) * NL + sub) * 2 + (part - 2)) * RB + col;
      // the first token of a logical page starts its statistics
      st16(dst, slot % p.logical == 0 ? k : fold16<DT>(ld16(dst), k, part == 2));
    }
  }
}

// One wave per (request, KV head) for 8- or 4-bit pages: lanes [0, LPR)
// quantize the new key row, lanes [LPR, 2 LPR) the value row (each group sits
// inside one DPP row, so its maximum is a DPP reduction); the other lanes
// idle.
template <int DT, int D, int BITS>
__global__ __launch_bounds__(kAppendWaves * kWave) void append_kv_fp8_kernel(AppendFp8Params p) {
  constexpr int LPR = D / 8;
  constexpr int RB = D * BITS / 8;  // code bytes per row
  constexpr int ES = DT == 0 ? 4 : 2;
  const int item = blockIdx.x * kAppendWaves + threadIdx.x / kWave;
  if (item >= p.S * p.Hkv) return;  // wave-uniform
  const int s = item / p.Hkv;
  const int kvh = item - s * p.Hkv;
  const int t = p.lens[s];
  if (t < 0 || t >= p.max_pages * p.P) return;  // full cache: nothing is written
  const int lp = t / p.P;
  const int slot = t - lp * p.P;
  const long long phys = p.table[(size_t)s * p.max_pages + lp];
  if (phys < 0 || phys >= p.NP) return;  // entry outside the pool: nothing is written
  const int lane = threadIdx.x % kWave;
  const int part = lane / LPR;  // 0 = key row, 1 = value row, else idle
  const int col = lane % LPR;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (part < 2) {
    const void* src = part == 0 ? p.k_new : p.v_new;
    load8<DT>(static_cast<const char*>(src) + (((size_t)s * p.Hkv + kvh) * D + col * 8) * ES, v);
  }
  float sc;
  uint2 c8 = make_uint2(0, 0);
  uint32_t c4 = 0;
  if constexpr (BITS == 8) c8 = quantize8<LPR>(v, sc);
  else c4 = quantize4<LPR>(v, sc);
  if (part < 2) {
    const size_t tile_id = p.head_major ? (size_t)kvh * p.NP + phys : (size_t)phys * p.Hkv + kvh;
    const size_t row = tile_id * p.P + slot;
    uint8_t* codes = part == 0 ? p.k_codes : p.v_codes;
    if constexpr (BITS == 8) *reinterpret_cast<uint2*>(codes + row * RB + col * 8) = c8;
    else *reinterpret_cast<uint32_t*>(codes + row * RB + col * 4) = c4;
    if (col == 0) (part == 0 ? p.k_scales : p.v_scales)[row] = sc;
  }
  // statistics of the logical page, folded from the full-precision key row
  // (as append_kv_kernel does for bf16 / fp32 pools)
  if (p.stats != nullptr && (p.select == nullptr || p.select[kvh] != 0)) {
    constexpr int RB = D * ES;
    constexpr int SL = RB / 16;  // 16-byte chunks per row
    const int NL = p.P / p.logical;
    const int sub = slot / p.logical;
    const char* k = static_cast<const char*>(p.k_new) + ((size_t)s * p.Hkv + kvh) * RB;
    char* base = static_cast<char*>(p.stats) + ((((size_t)kvh * p.NP + phys) * NL + sub) * 2) * RB;
    for (int cc = lane; cc < 2 * SL; cc += kWave) {
      const int which = cc / SL;  // 0 = kmax, 1 = kmin
      const size_t col16 = (size_t)(cc - which * SL) * 16;
      const uint4 kx = ld16(k + col16);
      char* dst = base + which * RB + col16;
      st16(dst, slot % p.logical == 0 ? kx : fold16<DT>(ld16(dst), kx, which == 0));
    }
  }
}

// One workgroup per (request, KV head).  Pages [0, n) with n = ceil(E / P),
// E = min(L + horizon, capacity), are split into contiguous per-thread
// chunks (thread order = page order); a block-wide exclusive scan of the
// per-chunk kept counts gives each chunk the ordinal of its first kept page.
// Bound j starts at the kept page of ordinal floor(j K / b): with up to 64
// pages per thread one thread per bound locates that page (chunk by binary
// search, page by the chunk's bit word); longer rows let every thread write
// the bounds whose ordinal falls in its chunk.
__global__ __launch_bounds__(kBoundsThreads) void split_bounds_kernel(BoundsParams p) {
  __shared__ int s_wave[kBoundsWaves];
  __shared__ int s_base[kBoundsThreads];        // first kept ordinal of each chunk
  __shared__ uint64_t s_bits[kBoundsThreads];   // kept flags of each chunk (packed rows)
  const int s = blockIdx.x / p.Hkv;
  const int kvh = blockIdx.x - s * p.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const long long cap = (long long)p.max_pages * p.P;
  const long long L = max(0, p.lens[s]);
  const int E = (int)min(L + p.horizon, cap);
  const int n = (E + p.P - 1) / p.P;
  const uint8_t* mrow = p.mask == nullptr ? nullptr : p.mask + ((size_t)s * p.Hkv + kvh) * p.max_pages;
  const int per = (n + kBoundsThreads - 1) / kBoundsThreads;
  const int c0 = min(n, tid * per);
  const int c1 = min(n, c0 + per);
  // Chunks of up to 64 pages (rows of up to 16384 pages): the chunk's kept
  // flags as one bit word, read with 64 independent loads issued together
  // (clamped to the row, so every load is in bounds) instead of one
  // dependent load per page; longer rows walk the mask page by page.
  const bool packed = per <= kBoundsBits;
  uint64_t bits = 0;
  if (packed && n > 0) {
    uint8_t v[kBoundsBits];
#pragma unroll
    for (int u = 0; u < kBoundsBits; ++u) v[u] = mrow == nullptr ? 1 : mrow[min(c0 + u, n - 1)];
#pragma unroll
    for (int u = 0; u < kBoundsBits; ++u) bits |= (c0 + u < c1 && v[u] != 0) ? 1ull << u : 0ull;
  }
  int cnt = 0;
  if (packed) cnt = __popcll(bits);
  else
    for (int lp = c0; lp < c1; ++lp) cnt += (mrow == nullptr || mrow[lp] != 0) ? 1 : 0;
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  int base = incl - cnt, K = 0;
#pragma unroll
  for (int w = 0; w < kBoundsWaves; ++w) {
    if (w < wave) base += s_wave[w];
    K += s_wave[w];
  }
  const int b = p.b;
  int32_t* out = p.bounds + ((size_t)s * p.Hkv + kvh) * (b + 1);
  if (tid == 0) {
    out[0] = 0;
    out[b] = E;
    if (K == 0)
      for (int j = 1; j < b; ++j) out[j] = E;
  }
  if (K == 0) return;
  if (packed) {
    // bound j (1 <= j < b) starts at the kept page of ordinal floor(j K / b):
    // one thread per bound finds the chunk holding that ordinal (binary
    // search over the chunks' first ordinals) and the page within it (the
    // matching set bit), one division per bound
    s_base[tid] = base;
    s_bits[tid] = bits;
    __syncthreads();
    for (int j = 1 + tid; j < b; j += kBoundsThreads) {
      const int t = (int)(((long long)j * K) / b);
      int lo = 0, hi = kBoundsThreads - 1;  // the last chunk whose first ordinal <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (s_base[mid] <= t) lo = mid;
        else hi = mid - 1;
      }
      uint64_t w = s_bits[lo];
      for (int r = t - s_base[lo]; r > 0; --r) w &= w - 1;  // drop the lower set bits
      out[j] = (lo * per + __builtin_ctzll(w)) * p.P;
    }
    return;
  }
  if (cnt == 0) return;
  int o = base;
  for (int lp = c0; lp < c1; ++lp) {
    if (mrow != nullptr && mrow[lp] == 0) continue;
    // the j >= 1 with floor(j K / b) == o: from ceil(o b / K) while it holds
    for (long long j = ((long long)o * b + K - 1) / K; j < b && (j * K) / b == o; ++j)
      if (j >= 1) out[j] = lp * p.P;
    ++o;
  }
}

}  // namespace

bool append_supported(int dtype, int D) { return (dtype == 0 || dtype == 1) && (D == 64 || D == 128); }

hipError_t launch_append_kv(const AppendParams& p, int dtype, int D, hipStream_t stream) {
  const long long items = (long long)p.S * p.Hkv;
  if (items < 1) return hipSuccess;
  const dim3 g((unsigned)((items + kAppendWaves - 1) / kAppendWaves)), b(kAppendWaves * kWave);
  if (dtype == 0 && D == 64) hipLaunchKernelGGL((append_kv_kernel<0, 64>), g, b, 0, stream, p);
  else if (dtype == 0 && D == 128) hipLaunchKernelGGL((append_kv_kernel<0, 128>), g, b, 0, stream, p);
  else if (dtype == 1 && D == 64) hipLaunchKernelGGL((append_kv_kernel<1, 64>), g, b, 0, stream, p);
  else if (dtype == 1 && D == 128) hipLaunchKernelGGL((append_kv_kernel<1, 128>), g, b, 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_append_kv_fp8(const AppendFp8Params& p, int dtype, int D, hipStream_t stream) {
  const long long items = (long long)p.S * p.Hkv;
  if (items < 1) return hipSuccess;
  const dim3 g((unsigned)((items + kAppendWaves - 1) / kAppendWaves)), b(kAppendWaves * kWave);
  if (p.bits == 4) {
    if (dtype == 0 && D == 64) hipLaunchKernelGGL((append_kv_fp8_kernel<0, 64, 4>), g, b, 0, stream, p);
    else if (dtype == 0 && D == 128) hipLaunchKernelGGL((append_kv_fp8_kernel<0, 128, 4>), g, b, 0, stream, p);
    else if (dtype == 1 && D == 64) hipLaunchKernelGGL((append_kv_fp8_kernel<1, 64, 4>), g, b, 0, stream, p);
    else if (dtype == 1 && D == 128) hipLaunchKernelGGL((append_kv_fp8_kernel<1, 128, 4>), g, b, 0, stream, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (p.bits != 8) return hipErrorInvalidValue;
  if (dtype == 0 && D == 64) hipLaunchKernelGGL((append_kv_fp8_kernel<0, 64, 8>), g, b, 0, stream, p);
  else if (dtype == 0 && D == 128) hipLaunchKernelGGL((append_kv_fp8_kernel<0, 128, 8>), g, b, 0, stream, p);
  else if (dtype == 1 && D == 64) hipLaunchKernelGGL((append_kv_fp8_kernel<1, 64, 8>), g, b, 0, stream, p);
  else if (dtype == 1 && D == 128) hipLaunchKernelGGL((append_kv_fp8_kernel<1, 128, 8>), g, b, 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_split_bounds(const BoundsParams& p, hipStream_t stream) {
  const long long rows = (long long)p.S * p.Hkv;
  if (rows < 1) return hipSuccess;
  hipLaunchKernelGGL(split_bounds_kernel, dim3((unsigned)rows), dim3(kBoundsThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace da
