// MicroAttention on the vector ALUs, for one query head per KV head (G = 1)
// and for fp32 K/V: per work item, the partial softmax statistics and
// unnormalised value sum of every query head of the KV head's group over the
// item's kept tokens:
//   m_j = max_i s_i,  e_j = sum_i exp(s_i - m_j),  MA_j = sum_i exp(s_i - m_j) v_i
// (Infinite-LLM page, section 方法细节, MicroAttention equations), with
// s_i = scale * (q . k_i).  Whole pages with a zero block-mask entry are
// neither loaded nor computed (LServe blog page, section 2.1.1).
//
// Work decomposition.  One 256-lane workgroup (4 waves) per work item.  The
// item's kept logical pages are compacted into an LDS list, then cut into
// 16-token slabs that the 4 waves take round-robin.  A slab of one KV head is
// contiguous in the pool ([page, head, slot, D] layout), so every wave-wide
// 16-byte load reads 1 KiB of consecutive bytes.  Each lane holds 16 bytes of
// one token row: a row of LPT = D*sizeof(elem)/16 consecutive lanes covers a
// token, so a wave load covers 64/LPT tokens ("rows").  Dot products are
// reduced inside each row with DPP; every row keeps its own online (m, e, MA)
// state -- the triple is closed under the aggregation rule, so rows never
// exchange maxima in the loop -- and rows and waves are combined once at the
// end of the item.
//
// Arithmetic: fp32 accumulation.  bf16 scores use v_dot2 (bf16 pairs, fp32
// accumulate); bf16 values are widened exactly by bit shifts.  fp8 (E4M3)
// keys are widened exactly to bf16 pairs for the same v_dot2 with the bf16
// query, fp8 values to fp32 by v_cvt_pk_f32_fp8; a token's K scale
// multiplies its dot product and its V scale its probability (per-row scales
// of the quantized pages).  Exponentials
// run in base 2 on raw dot products: exp(scale*(d - d_max)) =
// exp2((d - d_max) * scale*log2(e)); the reported m_j is scale * d_max.
#include <type_traits>

#include "micro_common.h"

namespace da {

hipError_t launch_micro_mfma(int dtype, int D, int G, const MicroParams& p, hipStream_t stream);
bool micro_mfma_supported(int dtype, int D, int G);

namespace {

// DT: 0 = fp32, 1 = bf16, 2 = fp8 E4M3 with per-row scales, 3 = fp4 E2M1
// with per-row scales (two codes per byte).  SL: tokens per slab (16; for
// quantized pages as many as the page size allows up to 8 KiB of K + V per
// slab -- 32 tokens of 8-bit rows, 64 of 4-bit rows -- so a slab moves as
// many bytes as a 16-token bf16 slab and as many stay in flight).
template <int DT, int D, int SL>
struct Layout {
  static constexpr int TOKB = DT == 0 ? 4 * D : DT == 1 ? 2 * D : DT == 2 ? D : D / 2;  // row bytes
  static constexpr int LPT = TOKB / 16;        // lanes per token row
  static constexpr int TPI = kWave / LPT;      // token rows per wave load
  static constexpr int EPL = DT == 0 ? 4 : DT == 1 ? 8 : DT == 2 ? 16 : 32;  // elements per lane
  static constexpr int QW = DT >= 2 ? EPL / 8 : 1;  // 16-byte words of the query per lane
  static constexpr int NI = SL / TPI;          // wave loads per slab per tensor
  static_assert(TPI * TOKB == kWave * 16, "wave load covers whole rows");
  static_assert(NI >= 1 && SL % TPI == 0, "slab covers whole wave loads");
};

template <int DT, int D, int SL>
struct Frag {
  uint4 k[Layout<DT, D, SL>::NI];
  uint4 v[Layout<DT, D, SL>::NI];
  float ks[Layout<DT, D, SL>::NI];  // fp8: K and V scales of this lane's token rows
  float vs[Layout<DT, D, SL>::NI];
};

template <int DT, int D, int G, int SL, bool kFused>
__global__ __launch_bounds__(kMicroThreads) void micro_kernel(MicroParams p) {
  using L = Layout<DT, D, SL>;
  __shared__ int s_phys[kPageCap];
  __shared__ int s_lp[kPageCap];
  __shared__ int s_cnt[kMicroWaves];
  __shared__ FinishLds<G, D> s_fin;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // the wave index is the same in every lane; saying so keeps the slab loop,
  // its page lookups and its address arithmetic on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int row = lane / L::LPT;
  const int chunk = lane % L::LPT;

  __shared__ int s_claim;
  for_each_item<kFused>(p, &s_claim, [&](int x) {
    const Item it = plan_item(p, x);
    const int s = it.s, kvh = it.kvh, h0 = kvh * G;
    const int t0 = it.t0, t1 = it.t1;
    const int P = p.P;
    const float c = p.scale * 1.4426950408889634f;  // scale * log2(e)

    // Query fragment of every head in the group: the lane's 16-byte column
    // (for quantized pages: the lane's EPL dims of the bf16 query, QW words
    // of 16 bytes).
    uint4 qv[G][L::QW];
  #pragma unroll
    for (int g = 0; g < G; ++g) {
      if constexpr (DT >= 2) {
        const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const char*>(p.q) +
                                                         (size_t)(s * p.Hq + h0 + g) * D * 2 +
                                                         (size_t)chunk * (L::EPL * 2));
  #pragma unroll
        for (int w = 0; w < L::QW; ++w) qv[g][w] = qp[w];
      } else {
        const char* qp = static_cast<const char*>(p.q) +
                         ((size_t)(s * p.Hq + h0 + g) * L::TOKB) + (size_t)chunk * 16;
        qv[g][0] = *reinterpret_cast<const uint4*>(qp);
      }
    }

    float m_[G], e_[G], acc[G][L::EPL];
  #pragma unroll
    for (int g = 0; g < G; ++g) {
      m_[g] = neg_inf();
      e_[g] = 0.f;
  #pragma unroll
      for (int k = 0; k < L::EPL; ++k) acc[g][k] = 0.f;
    }

    const Piece pc = plan_piece(p, it, s_cnt);
    if (pc.o0 < pc.o1) {
      const int32_t* trow = p.table + (size_t)s * p.max_pages;
      // slabs per page: P is a power of two, so slab sl is slab (sl & (spp - 1))
      // of kept page (sl >> spp_log)
      const int spp = P / SL;
      const int spp_log = __builtin_ctz(spp);
      // rows are counted from this KV head's first row: a page-major pool
      // [NP, Hkv, P, D] holds Hkv * P rows per page, a head-major pool
      // [Hkv, NP, P, D] holds P; the fp8 row scales share the row numbering
      const int page_rows = p.head_major ? P : p.Hkv * P;
      const size_t head_row = (size_t)kvh * (p.head_major ? (size_t)p.NP : (size_t)1) * P;
      const char* kbase = static_cast<const char*>(p.k) + head_row * L::TOKB + lane * 16;
      const char* vbase = static_cast<const char*>(p.v) + head_row * L::TOKB + lane * 16;
      // quantized pages: the scales of this lane's token rows (none for bf16 or fp32)
      const float* ksb = DT >= 2 ? p.ks + head_row + row : nullptr;
      const float* vsb = DT >= 2 ? p.vs + head_row + row : nullptr;

      // resume point of the page scan: without a mask, ordinal = page - pa
      int rlp = it.mrow ? it.pa : it.pa + pc.o0;
      int rord = it.mrow ? 0 : pc.o0;
      for (int w0 = pc.o0; w0 < pc.o1; w0 += kPageCap) {
        const int nk = compact_window(rlp, rord, it.pb, w0, min(pc.o1, w0 + kPageCap), it.mrow,
                                      trow, s_phys, s_lp, s_cnt);

        // ---- stream the piece's slabs: wave w takes slabs w, w+4, ... ----
        const int nslab = nk * spp;

        // where slab sl lives; the page ids are read from LDS as wave-uniform
        // values so that the offsets are computed on the scalar unit
        struct Pos {
          size_t row;  // the slab's first row (pool bytes: row * TOKB)
          int tb;      // logical token of the slab's first row
          bool whole;  // every row of the slab lies inside the split
        };
        auto pos = [&](int sl) {
          const int kp = sl >> spp_log;
          const int sub = sl & (spp - 1);
          const int phys = __builtin_amdgcn_readfirstlane(s_phys[kp]);
          const int lp = __builtin_amdgcn_readfirstlane(s_lp[kp]);
          Pos q;
          q.row = (size_t)phys * page_rows + sub * SL;
          q.tb = lp * P + sub * SL;
          q.whole = q.tb >= t0 && q.tb + SL <= t1;
          return q;
        };

        auto load = [&](int sl, Frag<DT, D, SL>& f) {
          const Pos q = pos(sl);
          const size_t off = q.row * L::TOKB;
          if (q.whole) {
  #pragma unroll
            for (int i = 0; i < L::NI; ++i) {
              f.k[i] = load_stream16(kbase + off + i * 1024);
              f.v[i] = load_stream16(vbase + off + i * 1024);
              if constexpr (DT >= 2) {
                f.ks[i] = ksb[q.row + i * L::TPI];
                f.vs[i] = vsb[q.row + i * L::TPI];
              }
            }
          } else {
  #pragma unroll
            for (int i = 0; i < L::NI; ++i) {
              const int t = q.tb + i * L::TPI + row;
              if (t >= t0 && t < t1) {
                f.k[i] = load_stream16(kbase + off + i * 1024);
                f.v[i] = load_stream16(vbase + off + i * 1024);
                if constexpr (DT >= 2) {
                  f.ks[i] = ksb[q.row + i * L::TPI];
                  f.vs[i] = vsb[q.row + i * L::TPI];
                }
              } else {
                // rows outside the split: zeros, never the (unread) slot's contents
                f.k[i] = make_uint4(0, 0, 0, 0);
                f.v[i] = make_uint4(0, 0, 0, 0);
                f.ks[i] = 0.f;
                f.vs[i] = 0.f;
              }
            }
          }
        };

        // One slab.  A slab cut by the split bounds differs only in its
        // scores: rows outside the split score -inf (weight 0), and their keys
        // and values were loaded as zeros.
        auto compute = [&](int sl, const Frag<DT, D, SL>& f) {
          const Pos q = pos(sl);

          // scores: dot[i][g] for this row's token of wave load i
          float dot[L::NI][G];
  #pragma unroll
          for (int i = 0; i < L::NI; ++i) {
  #pragma unroll
            for (int g = 0; g < G; ++g) {
              float d;
              const uint32_t w4[4] = {f.k[i].x, f.k[i].y, f.k[i].z, f.k[i].w};
              uint32_t qw[4 * L::QW];
  #pragma unroll
              for (int w = 0; w < L::QW; ++w) {
                qw[4 * w] = qv[g][w].x;
                qw[4 * w + 1] = qv[g][w].y;
                qw[4 * w + 2] = qv[g][w].z;
                qw[4 * w + 3] = qv[g][w].w;
              }
              if constexpr (DT == 3) {
                // codes widened to bf16 pairs (byte b of word w: dims 8w + 2b,
                // 8w + 2b + 1), then bf16 dot products with q
                d = 0.f;
  #pragma unroll
                for (int w = 0; w < 4; ++w) {
                  d = dot2_bf16(fp4x2_to_bf16x2<0>(w4[w]), qw[4 * w], d);
                  d = dot2_bf16(fp4x2_to_bf16x2<1>(w4[w]), qw[4 * w + 1], d);
                  d = dot2_bf16(fp4x2_to_bf16x2<2>(w4[w]), qw[4 * w + 2], d);
                  d = dot2_bf16(fp4x2_to_bf16x2<3>(w4[w]), qw[4 * w + 3], d);
                }
              } else if constexpr (DT == 2) {
                // codes widened to bf16 pairs, then bf16 dot products with q
                d = 0.f;
  #pragma unroll
                for (int w = 0; w < 4; ++w) {
                  d = dot2_bf16(fp8x2_to_bf16x2<false>(w4[w]), qw[2 * w], d);
                  d = dot2_bf16(fp8x2_to_bf16x2<true>(w4[w]), qw[2 * w + 1], d);
                }
              } else if constexpr (DT == 1) {
                d = dot2_bf16(w4[0], qw[0], 0.f);
                d = dot2_bf16(w4[1], qw[1], d);
                d = dot2_bf16(w4[2], qw[2], d);
                d = dot2_bf16(w4[3], qw[3], d);
              } else {
                d = __builtin_bit_cast(float, w4[0]) * __builtin_bit_cast(float, qw[0]);
                d = fmaf(__builtin_bit_cast(float, w4[1]), __builtin_bit_cast(float, qw[1]), d);
                d = fmaf(__builtin_bit_cast(float, w4[2]), __builtin_bit_cast(float, qw[2]), d);
                d = fmaf(__builtin_bit_cast(float, w4[3]), __builtin_bit_cast(float, qw[3]), d);
              }
              dot[i][g] = group_sum<L::LPT>(d);
              if constexpr (DT >= 2) dot[i][g] *= f.ks[i];
            }
          }
          if (!q.whole) {  // wave-uniform branch
  #pragma unroll
            for (int i = 0; i < L::NI; ++i) {
              const int t = q.tb + i * L::TPI + row;
              const bool valid = t >= t0 && t < t1;
  #pragma unroll
              for (int g = 0; g < G; ++g) dot[i][g] = valid ? dot[i][g] : neg_inf();
            }
          }

          // online softmax update, once per slab
          float pw[L::NI][G];
  #pragma unroll
          for (int g = 0; g < G; ++g) {
            float mx = m_[g];
  #pragma unroll
            for (int i = 0; i < L::NI; ++i) mx = fmaxf(mx, dot[i][g]);
            const float ms = mx != neg_inf() ? mx : 0.f;
            const float alpha = fast_exp2((m_[g] - ms) * c);
            const float nmc = -ms * c;
            float sum = 0.f;
  #pragma unroll
            for (int i = 0; i < L::NI; ++i) {
              const float w = fast_exp2(fmaf(dot[i][g], c, nmc));
              pw[i][g] = w;
              sum += w;
            }
            e_[g] = fmaf(e_[g], alpha, sum);
            m_[g] = mx;
  #pragma unroll
            for (int k = 0; k < L::EPL; ++k) acc[g][k] *= alpha;
          }

          // weighted value sum
  #pragma unroll
          for (int i = 0; i < L::NI; ++i) {
            float vf[L::EPL];
            if constexpr (DT == 3) {
              const uint32_t w4[4] = {f.v[i].x, f.v[i].y, f.v[i].z, f.v[i].w};
  #pragma unroll
              for (int w = 0; w < 4; ++w) fp4x8_to_f32(w4[w], vf + 8 * w);
            } else if constexpr (DT == 2) {
              const uint32_t w4[4] = {f.v[i].x, f.v[i].y, f.v[i].z, f.v[i].w};
  #pragma unroll
              for (int w = 0; w < 4; ++w) fp8x4_to_f32(w4[w], vf + 4 * w);
            } else if constexpr (DT == 1) {
              const uint32_t w4[4] = {f.v[i].x, f.v[i].y, f.v[i].z, f.v[i].w};
  #pragma unroll
              for (int k = 0; k < 4; ++k) {
                vf[2 * k] = bf16_lo(w4[k]);
                vf[2 * k + 1] = bf16_hi(w4[k]);
              }
            } else {
              vf[0] = __builtin_bit_cast(float, f.v[i].x);
              vf[1] = __builtin_bit_cast(float, f.v[i].y);
              vf[2] = __builtin_bit_cast(float, f.v[i].z);
              vf[3] = __builtin_bit_cast(float, f.v[i].w);
            }
  #pragma unroll
            for (int g = 0; g < G; ++g) {
              const float pv = DT >= 2 ? pw[i][g] * f.vs[i] : pw[i][g];
  #pragma unroll
              for (int k = 0; k < L::EPL; ++k) acc[g][k] = fmaf(pv, vf[k], acc[g][k]);
            }
          }
        };

        constexpr int W = kMicroWaves;
        if constexpr (SL == kSlab) {
          // two slabs in flight ahead of the one being computed; the three
          // fragments take turns (no register copies, which would have to
          // wait for the loads in flight)
          Frag<DT, D, SL> f0, f1, f2;
          int sl = wave;
          if (sl < nslab) load(sl, f0);
          if (sl + W < nslab) load(sl + W, f1);
          while (sl < nslab) {
            if (sl + 2 * W < nslab) load(sl + 2 * W, f2);
            compute(sl, f0);
            sl += W;
            if (sl >= nslab) break;
            if (sl + 2 * W < nslab) load(sl + 2 * W, f0);
            compute(sl, f1);
            sl += W;
            if (sl >= nslab) break;
            if (sl + 2 * W < nslab) load(sl + 2 * W, f1);
            compute(sl, f2);
            sl += W;
          }
        } else {
          // double-length fp8 slabs: one in flight ahead keeps the register
          // budget of two waves per SIMD
          Frag<DT, D, SL> fa, fb;
          int sl = wave;
          if (sl < nslab) load(sl, fa);
          while (sl < nslab) {
            if (sl + W < nslab) load(sl + W, fb);
            compute(sl, fa);
            sl += W;
            if (sl >= nslab) break;
            if (sl + W < nslab) load(sl + W, fa);
            compute(sl, fb);
            sl += W;
          }
        }
        __syncthreads();  // the page list is rewritten by the next batch
      }
    }

    // ---- combine the rows of each wave (lanes l and l ^ (k * LPT)) ----
  #pragma unroll
    for (int off = L::LPT; off < kWave; off <<= 1) {
  #pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mo = __shfl_xor(m_[g], off, kWave);
        const float eo = __shfl_xor(e_[g], off, kWave);
        const float M = fmaxf(m_[g], mo);
        const float Ms = (M == neg_inf()) ? 0.f : M;
        const float a = fast_exp2((m_[g] - Ms) * c);
        const float b = fast_exp2((mo - Ms) * c);
        e_[g] = e_[g] * a + eo * b;
  #pragma unroll
        for (int k = 0; k < L::EPL; ++k) {
          const float ao = __shfl_xor(acc[g][k], off, kWave);
          acc[g][k] = acc[g][k] * a + ao * b;
        }
        m_[g] = M;
      }
    }
    finish_item<G, D, L::LPT, L::EPL, kFused>(p, it, s_fin, m_, e_, acc, c);
  });
}

// Pieces of at least this many bytes of K and V run one workgroup per CU.
constexpr long long kLongPieceBytes = 4LL << 20;

// Resident workgroups per CU, chosen per launch (0: as many as registers
// allow, three for the bf16 instances).  Fewer, deeper streams read HBM
// faster once a CU's workgroups need not hide each other's per-item fixed
// cost: one per CU for long pieces of bf16, fp32 or 8-bit rows (C4: 2390
// against 2435 us, over 8-bit pages 1229 against 1256), two on the
// persistent work queues (C3: 887-896 against 904-911 us), as many as fit
// for short pieces (C2: 165 us, 197 with one per CU) and for 4-bit rows,
// whose arithmetic per byte one workgroup per CU cannot cover (C4 over
// 4-bit pages: 741 us with one, 668 with three).  The schedule is settled
// first, with the uncapped slots, so the cap does not move a launch between
// the two schedules.
template <int DT, int D, int G, int SL = kSlab>
hipError_t launch_one(const MicroParams& p0, hipStream_t stream) {
  using L = Layout<DT, D, SL>;
  const auto plain = micro_kernel<DT, D, G, SL, false>;
  MicroParams p = p0;
  int cap = 0;
  const int slots = resident_slots(reinterpret_cast<const void*>(plain), 0);
  const bool persistent = p.queue != nullptr && slots > 0 &&
                          (p.schedule == 2 ||
                           (p.schedule == 0 && p.n_items > kPersistentFactor * slots));
  if (persistent) {
    cap = 2;
    p.schedule = 2;
  } else {
    const long long row = 2LL * L::TOKB + (DT >= 2 ? 8 : 0);  // K and V (and their scales)
    if (DT <= 2 && (long long)p.piece_pages * p.P * row >= kLongPieceBytes) cap = 1;
    if (p.schedule == 0) p.schedule = 1;
  }
  return launch_micro_step<D>(plain, micro_kernel<DT, D, G, SL, true>, cap, p, stream);
}

template <int DT, int D>
hipError_t dispatch_g(int G, const MicroParams& p, hipStream_t stream) {
  switch (G) {
    case 1: return launch_one<DT, D, 1>(p, stream);
    case 2: return launch_one<DT, D, 2>(p, stream);
    case 4: return launch_one<DT, D, 4>(p, stream);
    case 8: return launch_one<DT, D, 8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool micro_supported(int dtype, int D, int G) {
  if (D != 64 && D != 128) return false;
  if (dtype == 2 || dtype == 3) return G == 1 || micro_mfma_supported(dtype, D, G);
  return (dtype == 0 || dtype == 1) && (G == 1 || G == 2 || G == 4 || G == 8);
}

long long micro_target_items(int dtype, int D, int G) {
  return micro_mfma_supported(dtype, D, G) ? 4096 : 1024;
}

// bf16 and fp8 with grouped query heads go to the matrix-core kernel; one
// query head per KV head and fp32 K/V stay on the vector ALUs.
hipError_t launch_micro(int dtype, int D, int G, const MicroParams& p, hipStream_t stream) {
  if (!micro_supported(dtype, D, G)) return hipErrorInvalidValue;
  if (micro_mfma_supported(dtype, D, G)) return launch_micro_mfma(dtype, D, G, p, stream);
  if (dtype == 0) return D == 64 ? dispatch_g<0, 64>(G, p, stream) : dispatch_g<0, 128>(G, p, stream);
  if (dtype == 2) {  // fp8 pages: one query head per KV head here, groups on the matrix cores
    if (p.P % 32 == 0)
      return D == 64 ? launch_one<2, 64, 1, 32>(p, stream) : launch_one<2, 128, 1, 32>(p, stream);
    return D == 64 ? launch_one<2, 64, 1>(p, stream) : launch_one<2, 128, 1>(p, stream);
  }
  if (dtype == 3) {  // fp4 pages: slabs of up to 64 tokens (8 KiB of K + V at D = 128)
    if (D == 64) {  // 32 rows per wave load: pages of 32 tokens or more
      if (p.P % 64 == 0) return launch_one<3, 64, 1, 64>(p, stream);
      if (p.P % 32 == 0) return launch_one<3, 64, 1, 32>(p, stream);
      return hipErrorInvalidValue;
    }
    if (p.P % 64 == 0) return launch_one<3, 128, 1, 64>(p, stream);
    if (p.P % 32 == 0) return launch_one<3, 128, 1, 32>(p, stream);
    return launch_one<3, 128, 1, 16>(p, stream);
  }
  return D == 64 ? dispatch_g<1, 64>(G, p, stream) : dispatch_g<1, 128>(G, p, stream);
}

}  // namespace da
