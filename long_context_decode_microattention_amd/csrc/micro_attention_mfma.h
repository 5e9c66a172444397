// MicroAttention on the matrix cores, for bf16, FP8 or FP4 K/V with G = 2, 4
// or 8 query heads per KV head (grouped-query attention).  Same per-item
// result as the vector kernel -- m_j, e_j and MA_j of the MicroAttention
// equations (Infinite-LLM page, section 方法细节) for every query head of the
// group -- with the page list, slabs and block-mask skipping of that kernel.
//
// With G query heads per KV head the scores and the value sums are small
// dense contractions, and on the vector ALUs they cost about 3 instructions
// per KV byte, too close to the issue budget to keep HBM saturated.  Per
// 16-token slab a wave instead runs:
//
//   scores   S[h][t] = q_h . k_t on v_mfma_f32_16x16x32_bf16: A = the query
//            heads (16 rows, G used), B = the slab's keys (16 columns), K =
//            D in 32-wide steps.  The B operand wants lane l to hold 8
//            consecutive dims of token l%16, so each key load reads 64
//            contiguous bytes of 16 token rows (the dims are visited in the
//            order chunk = 4*step + l/16; q uses the same order).  Lane l,
//            register i receives S[4*(l/16) + i][l % 16].
//   softmax  per-head slab maxima by DPP reductions over the 16 lanes of a
//            row, read out as wave-uniform values; the running maximum is
//            per wave, so the value accumulators are rescaled only when a
//            head's maximum rises (wave-uniform branch).
//   values   (bf16 pages with G <= 4, and any page type at D = 64) on
//            v_mfma_f32_4x4x1_16b_f32 (16 blocks of 4x4, K = 1): block
//            b = l/4 takes A = p of heads 0..3 from lanes 4b..4b+3 and B = one
//            value element from each of its 4 lanes, so the values are used
//            in the coalesced layout of the vector kernel (lane l holds 8
//            dims of token row l/LPT) and every lane ends up with its own 8
//            dims x 4 heads, all four block rows useful for G >= 4.  The
//            probabilities move from the score layout to that operand
//            layout through an SL x G float scratch in LDS per wave.
//
// fp8 (E4M3) and fp4 (E2M1) pages with per-row scales take the same score
// path: a lane's key codes (8 dims per score step, the steps of a lane now
// contiguous: dims grp*D/4 + 8*step, q in the same order) are widened exactly
// to bf16 for the score MFMA and the score column is multiplied by its
// token's K scale.  A token's V scale multiplies its probabilities in the
// score layout (where the lane of token `col` loads it next to the K scale),
// so the value operand arrives in LDS already scaled; the exp-sums take the
// unscaled probabilities.  Their value sums at D = 128 run on the dense bf16
// MFMA instead (dense_values below): with 4 or 8 times fewer bytes per token
// than bf16 pages, the 4x4x1 value product took 20-30% of every SIMD's
// cycles on the matrix pipe.  An 8-bit slab is 32 tokens with pages of 32
// tokens or more (G <= 4), two score groups of 16 under one running-max
// update and one LDS round trip (8 KiB of K + V, like a bf16 slab); a 4-bit
// slab is 64 tokens (four score groups) likewise.  With G <= 4 such a slab's
// softmax runs on its scores packed one token per lane (lane shuffles gather
// the groups, whose heads fill one row of lanes each), so the scales, mask,
// exponentials and the probability store cost one pass per token; each lane
// then loads its own token's K and V scales.
//
// The kernel template lives in this header; micro_attention_mfma.hip launches
// the bf16 instances, micro_attention_mfma_fp8.hip the 8-bit ones and
// micro_attention_mfma_fp4.hip the 4-bit ones, the last two built with
// different floating-point flags.
#pragma once

#include "micro_common.h"

namespace da {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// DT: 1 = bf16 pages, 2 = fp8 E4M3 pages, 3 = fp4 E2M1 pages (two codes per
// byte), the quantized ones with per-row scales.  Either way a value lane
// holds 8 dims of one token row (LPT lanes per row).  A slab is SL = 16, 32
// or 64 tokens: NG score groups of 16 tokens (token 16*g + col of group g in
// score column col).
template <int DT, int D, int SL>
struct MLayout {
  static constexpr int TOKB = DT == 1 ? D * 2 : DT == 2 ? D : D / 2;  // token row bytes
  static constexpr int LPT = D / 8;                // value lanes per token row
  static constexpr int TPI = kWave / LPT;          // token rows per value load
  static constexpr int NI = SL / TPI;              // value loads per slab
  static constexpr int NG = SL / 16;               // score groups per slab
  static constexpr int KS = D / 32;                // score k-steps
  static constexpr int KL = DT == 1 ? KS : KS / 2; // 16-byte key loads per lane (bf16, fp8)
  static constexpr int VB = DT == 1 ? 16 : DT == 2 ? 8 : 4;  // value bytes per lane per load
  static constexpr int EPL = 8;                    // elements per lane
};

template <int DT, int D, int SL>
struct MFrag {
  using L = MLayout<DT, D, SL>;
  uint4 k[DT == 3 ? 1 : L::NG][L::KL];
  uint32_t k4[DT == 3 ? L::NG : 1][L::KS];  // fp4 keys: 8 codes (one score step) per word
  uint4 v[DT == 1 ? L::NI : 1];   // bf16 values
  uint2 v8[DT == 2 ? L::NI : 1];  // fp8 values
  uint32_t v4[DT == 3 ? L::NI : 1];  // fp4 values
  float ksc[L::NG];               // quantized pages: K scale of token 16*g + col (packed
                                  // softmax: ksc[0] holds token `lane`'s)
  float vsc[L::NG];               // quantized pages: V scale, likewise
};

// Eight E2M1 codes (one word) -> eight bf16 values (four words), exactly.
__device__ __forceinline__ uint4 fp4x8_to_bf16x8(uint32_t w) {
  return make_uint4(fp4x2_to_bf16x2<0>(w), fp4x2_to_bf16x2<1>(w), fp4x2_to_bf16x2<2>(w),
                    fp4x2_to_bf16x2<3>(w));
}

__device__ __forceinline__ uint32_t load_stream4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// Eight E4M3 codes (two words) -> eight bf16 values (four words), exactly.
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return make_uint4(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                    fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1));
}

__device__ __forceinline__ uint2 load_stream8(const void* p) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(t.x, t.y);
}

// A lane's KS words of fp4 key codes (4 * KS contiguous bytes).
template <int KS>
__device__ __forceinline__ void load_key_words(const char* p, uint32_t (&w)[KS]) {
  static_assert(KS == 2 || KS == 4, "key steps");
  if constexpr (KS == 4) {
    const uint4 t = load_stream16(p);
    w[0] = t.x;
    w[1] = t.y;
    w[2] = t.z;
    w[3] = t.w;
  } else {
    const uint2 t = load_stream8(p);
    w[0] = t.x;
    w[1] = t.y;
  }
}

__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  x = fmaxf(x, dpp<kDppRowMirror>(x));
  return x;
}

__device__ __forceinline__ float lane_value(float x, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), src));
}

// Value product at D = 128 on the dense bf16 MFMA: over quantized pages, and
// over bf16 pages with G = 8 (whose 4x4x1 accumulators, 64 registers, left
// too few for the slabs in flight).
//
// A lane's value loads already hold what a B operand wants: load i gives lane
// l the 8 dims 8*(l%16) .. +7 of token 4i + l/16, so over a block of KB = 32
// (or 16) tokens the lane holds, for each of its dims, KB/4 tokens.  Taking
// column n = l%16 as dim 8n + e, v_mfma_f32_16x16x32_bf16 number e (e = 0..7)
// sums the block for dims 8n + e: its B operand is element e of the lane's 8
// loads, gathered into bf16 pairs (bf16 values by a half-word permutation;
// codes of two tokens side by side by a byte or nibble permutation, then one
// exact widening each), and its A operand is
// the probabilities of the same tokens, read from the per-wave LDS buffer
// where they are stored head-major with each block's tokens ordered by
// (token % 4, token / 4), so that a lane's KB/4 values are contiguous.
//
// The probabilities are fp32 (with the token's V scale folded in).  Each is
// split into a bf16 high part and the bf16 rounding of the remainder (the
// pair carries 16 significant bits, relative error <= 2^-17); with G query
// heads the high parts fill A rows 0 .. G-1 and the low parts rows G ..
// 2G-1 of the same instruction (16 rows, G <= 8), so the split costs no extra
// matrix work: output row r accumulates head r % G, and the two rows of a
// head are added once per item.  Per 32 tokens: 8 MFMA (128 busy cycles)
// instead of 64 v_mfma_f32_4x4x1f32 (512).
template <int DT, int D, int G>
inline constexpr bool kDenseValues = D == 128 && (DT >= 2 || (DT == 1 && G == 8));

template <int DT, int D, int G, int SL>
__device__ __forceinline__ void dense_values(const float* sp, const MFrag<DT, D, SL>& f,
                                             f32x4_t (&acc)[8]) {
  static_assert(kDenseValues<DT, D, G>, "dense value product: D = 128, quantized pages or G = 8");
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  constexpr int KB = SL < 32 ? SL : 32;  // tokens per block
  constexpr int KK = KB / 4;             // operand elements per lane
  constexpr int KW = KK / 2;             // operand words per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int row = lane & 15;
  const float* src = sp + (row % G) * SL + KK * (lane >> 4);
#pragma unroll
  for (int b = 0; b < SL / KB; ++b) {
    // A: probabilities of head row % G, tokens KB*b + 4*kk + lane/16
    float x[KK];
#pragma unroll
    for (int q = 0; q < KK / 4; ++q) {
      const float4 t = *reinterpret_cast<const float4*>(src + KB * b + 4 * q);
      x[4 * q] = t.x;
      x[4 * q + 1] = t.y;
      x[4 * q + 2] = t.z;
      x[4 * q + 3] = t.w;
    }
    uint32_t a[KW];
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      const f32x2_t v = {x[2 * j], x[2 * j + 1]};
      const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
      const f32x2_t rest = {x[2 * j] - bf16_lo(hi), x[2 * j + 1] - bf16_hi(hi)};
      const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(rest, bf16x2_t));
      a[j] = row < G ? hi : (row < 2 * G ? lo : 0u);
    }
    // B of instruction e: element e of loads KK*b + 2j and KK*b + 2j + 1 in
    // word j.  The codes of each load pair are first interleaved (pk[.][j]),
    // then widened one instruction's operand at a time, so that few operand
    // words are live at once.
    auto mfma = [&](int e, const uint32_t (&bw)[KW]) {
      if constexpr (KB == 32) {
        const uint4 av = make_uint4(a[0], a[1], a[2], a[3]);
        const uint4 bq = make_uint4(bw[0], bw[1], bw[2], bw[3]);
        acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                        __builtin_bit_cast(bf16x8_t, bq), acc[e], 0,
                                                        0, 0);
      } else {
        const uint2 av = make_uint2(a[0], a[1]);
        const uint2 bq = make_uint2(bw[0], bw[1]);
        acc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, av),
                                                          __builtin_bit_cast(s16x4_t, bq), acc[e],
                                                          0, 0, 0);
      }
    };
    if constexpr (DT == 1) {
      // element e of each bf16 load: half e % 2 of word e / 2; the two loads'
      // halves side by side
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t bw[KW];
#pragma unroll
        for (int j = 0; j < KW; ++j) {
          const uint4& va = f.v[KK * b + 2 * j];
          const uint4& vc = f.v[KK * b + 2 * j + 1];
          const int w = e >> 1;
          const uint32_t wa = w == 0 ? va.x : (w == 1 ? va.y : (w == 2 ? va.z : va.w));
          const uint32_t wc = w == 0 ? vc.x : (w == 1 ? vc.y : (w == 2 ? vc.z : vc.w));
          bw[j] = __builtin_amdgcn_perm(wc, wa, (e & 1) ? 0x07060302u : 0x05040100u);
        }
        mfma(e, bw);
      }
    } else if constexpr (DT == 2) {
      // word w of each load: bytes (a_q, c_q) side by side -> dims 4w + q
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        uint32_t pk[2][KW];
#pragma unroll
        for (int j = 0; j < KW; ++j) {
          const int i0 = KK * b + 2 * j;
          const uint32_t wa = w ? f.v8[i0].y : f.v8[i0].x;
          const uint32_t wc = w ? f.v8[i0 + 1].y : f.v8[i0 + 1].x;
          pk[0][j] = __builtin_amdgcn_perm(wc, wa, 0x05010400u);  // a0 c0 a1 c1
          pk[1][j] = __builtin_amdgcn_perm(wc, wa, 0x07030602u);  // a2 c2 a3 c3
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t bw[KW];
#pragma unroll
          for (int j = 0; j < KW; ++j)
            bw[j] = (q & 1) ? fp8x2_to_bf16x2<true>(pk[q >> 1][j]) : fp8x2_to_bf16x2<false>(pk[q >> 1][j]);
          mfma(4 * w + q, bw);
        }
      }
    } else {
      // byte q: the (a, c) codes of element 2q (even word) or 2q + 1 (odd word)
      uint32_t pk[2][KW];
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        const uint32_t wa = f.v4[KK * b + 2 * j], wc = f.v4[KK * b + 2 * j + 1];
        pk[0][j] = (wa & 0x0F0F0F0Fu) | ((wc & 0x0F0F0F0Fu) << 4);
        pk[1][j] = ((wa >> 4) & 0x0F0F0F0Fu) | (wc & 0xF0F0F0F0u);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t bw[KW];
#pragma unroll
        for (int j = 0; j < KW; ++j) {
          const uint32_t src = pk[e & 1][j];
          switch (e >> 1) {
            case 0: bw[j] = fp4x2_to_bf16x2<0>(src); break;
            case 1: bw[j] = fp4x2_to_bf16x2<1>(src); break;
            case 2: bw[j] = fp4x2_to_bf16x2<2>(src); break;
            default: bw[j] = fp4x2_to_bf16x2<3>(src); break;
          }
        }
        mfma(e, bw);
      }
    }
  }
}

// Two waves per SIMD: the register budget that holds the prefetched slab, the
// query operand and the accumulators without spilling (measured faster than
// three waves with spills).
template <int DT, int D, int G, int SL, bool kFused>
__global__ __launch_bounds__(kMicroThreads)
__attribute__((amdgpu_waves_per_eu(2))) void micro_mfma_kernel(MicroParams p) {
  using L = MLayout<DT, D, SL>;
  constexpr int HS = (G + 3) / 4;  // groups of 4 heads (score rows / value head sets)
  static_assert(G == 2 || G == 4 || G == 8, "group size");
  constexpr bool kDense = kDenseValues<DT, D, G>;
  // softmax on the scores packed one token per lane (at most 4 heads, 2 or 4
  // score groups per slab)
  constexpr bool kPacked = kDense && G <= 4 && L::NG >= 2;
  constexpr int KB = SL < 32 ? SL : 32;  // tokens per dense value block
  __shared__ int s_phys[kPageCap];
  __shared__ int s_lp[kPageCap];
  __shared__ int s_cnt[kMicroWaves];
  __shared__ __align__(16) float s_p[kMicroWaves][SL * G];
  __shared__ FinishLds<G, D> s_fin;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // the wave index is the same in every lane; saying so keeps the slab loop,
  // its page lookups and its address arithmetic on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 15;  // score column: token within a score group
  const int grp = lane >> 4;  // score row group: heads 4*grp .. 4*grp+3
  const int vrow = lane / L::LPT;
  const int quad = lane & 3;  // head within a 4x4 block of the value product

  __shared__ int s_claim;
  for_each_item<kFused>(p, &s_claim, [&](int x) {
    const Item it = plan_item(p, x);
    const int s = it.s, kvh = it.kvh, h0 = kvh * G;
    const int t0 = it.t0, t1 = it.t1;
    const int P = p.P;
    const float c = p.scale * 1.4426950408889634f;  // scale * log2(e)

    // score operand A: lane l -> head l%16 (zero beyond G), 8 bf16 dims per
    // step: chunk 4*step + l/16 (bf16 pages) or chunk KS*(l/16) + step (fp8)
    uint4 qa[L::KS];
  #pragma unroll
    for (int st = 0; st < L::KS; ++st) {
      qa[st] = make_uint4(0, 0, 0, 0);
      if (col < G) {
        const int chunk8 = DT == 1 ? 4 * st + grp : L::KS * grp + st;
        const char* qp = static_cast<const char*>(p.q) + (size_t)(s * p.Hq + h0 + col) * D * 2 +
                         (size_t)chunk8 * 16;
        qa[st] = *reinterpret_cast<const uint4*>(qp);
      }
    }

    float m_h[G];        // running raw-dot maximum per head (wave-uniform)
    float e_l[4];        // per-lane exp-sums: token column `col`, heads 4*grp + i (packed:
                         // token `lane` of each slab, head i)
    // value sums.  4x4 blocks: acc[hs][k] register i = head 4*hs + i, dim k
    // of the lane's 8.  Dense form: acc[0][e] = the 16 x 16 output tile of
    // dims 8n + e (column n = lane % 16); register i holds row 4*(lane/16) + i
    // (rows < G: the high parts of the probabilities, G .. 2G - 1: the low
    // parts, the rest zero)
    f32x4_t acc[kDense ? 1 : HS][8];
  #pragma unroll
    for (int h = 0; h < G; ++h) m_h[h] = neg_inf();
  #pragma unroll
    for (int i = 0; i < 4; ++i) e_l[i] = 0.f;
  #pragma unroll
    for (int hs = 0; hs < (kDense ? 1 : HS); ++hs)
  #pragma unroll
      for (int k = 0; k < 8; ++k) acc[hs][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};

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
      // key lane: token col; bf16: 16 bytes per step at 64*step + 16*grp;
      // fp8: 8*KS contiguous bytes at 8*KS*grp
      const char* kbase = static_cast<const char*>(p.k) + head_row * L::TOKB +
                          (size_t)col * L::TOKB +
                          (size_t)grp * (DT == 1 ? 16 : DT == 2 ? 8 * L::KS : 4 * L::KS);
      const char* vbase = static_cast<const char*>(p.v) + head_row * L::TOKB + lane * L::VB;
      // fp8: the K and V scales of the key lane's token (no scales for bf16)
      const float* ksb = DT >= 2 ? p.ks + head_row + col : nullptr;
      const float* vsb = DT >= 2 ? p.vs + head_row + col : nullptr;
      // packed softmax: lane l takes token l of the slab (the last one past SL)
      const int tl = lane < SL ? lane : SL - 1;
      const float* ksp = DT >= 2 ? p.ks + head_row + tl : nullptr;
      const float* vsp = DT >= 2 ? p.vs + head_row + tl : nullptr;

      // resume point of the page scan: without a mask, ordinal = page - pa
      int rlp = it.mrow ? it.pa : it.pa + pc.o0;
      int rord = it.mrow ? 0 : pc.o0;
      for (int w0 = pc.o0; w0 < pc.o1; w0 += kPageCap) {
        const int nk = compact_window(rlp, rord, it.pb, w0, min(pc.o1, w0 + kPageCap), it.mrow,
                                      trow, s_phys, s_lp, s_cnt);
        const int nslab = nk * spp;

        // key load j of a lane: bf16 64*j (one score step), fp8 16*j (two steps)
        constexpr int KSTRIDE = DT == 1 ? 64 : 16;
        constexpr int VSTRIDE = L::TPI * L::TOKB;  // bytes per value load

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

        auto load = [&](int sl, MFrag<DT, D, SL>& f) {
          const Pos q = pos(sl);
          const size_t off = q.row * L::TOKB;
          if (q.whole) {
  #pragma unroll
            for (int g = 0; g < L::NG; ++g) {
              if constexpr (DT == 3) {
                load_key_words<L::KS>(kbase + off + g * 16 * L::TOKB, f.k4[g]);
              } else {
  #pragma unroll
                for (int j = 0; j < L::KL; ++j)
                  f.k[g][j] = load_stream16(kbase + off + g * 16 * L::TOKB + j * KSTRIDE);
              }
              if constexpr (DT >= 2 && !kPacked) {
                f.ksc[g] = ksb[q.row + 16 * g];
                f.vsc[g] = vsb[q.row + 16 * g];
              }
            }
            if constexpr (kPacked) {  // the scales of token `lane` of the slab
              f.ksc[0] = ksp[q.row];
              f.vsc[0] = vsp[q.row];
            }
  #pragma unroll
            for (int i = 0; i < L::NI; ++i) {
              if constexpr (DT == 1) {
                f.v[i] = load_stream16(vbase + off + i * VSTRIDE);
              } else if constexpr (DT == 2) {
                f.v8[i] = load_stream8(vbase + off + i * VSTRIDE);
              } else {
                f.v4[i] = load_stream4(vbase + off + i * VSTRIDE);
              }
            }
          } else {  // rows outside the split read as zeros (and zero scales)
  #pragma unroll
            for (int g = 0; g < L::NG; ++g) {
              const int tk = q.tb + 16 * g + col;
              const bool kok = tk >= t0 && tk < t1;
              if constexpr (DT == 3) {
                if (kok) {
                  load_key_words<L::KS>(kbase + off + g * 16 * L::TOKB, f.k4[g]);
                } else {
  #pragma unroll
                  for (int st = 0; st < L::KS; ++st) f.k4[g][st] = 0;
                }
              } else {
  #pragma unroll
                for (int j = 0; j < L::KL; ++j)
                  f.k[g][j] = kok ? load_stream16(kbase + off + g * 16 * L::TOKB + j * KSTRIDE)
                                  : make_uint4(0, 0, 0, 0);
              }
              if constexpr (DT >= 2 && !kPacked) {
                f.ksc[g] = kok ? ksb[q.row + 16 * g] : 0.f;
                f.vsc[g] = kok ? vsb[q.row + 16 * g] : 0.f;
              }
            }
            if constexpr (kPacked) {
              const int tk = q.tb + lane;
              const bool kok = lane < SL && tk >= t0 && tk < t1;
              f.ksc[0] = kok ? ksp[q.row] : 0.f;
              f.vsc[0] = kok ? vsp[q.row] : 0.f;
            }
  #pragma unroll
            for (int i = 0; i < L::NI; ++i) {
              const int tv = q.tb + i * L::TPI + vrow;
              const bool vok = tv >= t0 && tv < t1;
              if constexpr (DT == 1) {
                f.v[i] = vok ? load_stream16(vbase + off + i * VSTRIDE) : make_uint4(0, 0, 0, 0);
              } else if constexpr (DT == 2) {
                f.v8[i] = vok ? load_stream8(vbase + off + i * VSTRIDE) : make_uint2(0, 0);
              } else {
                f.v4[i] = vok ? load_stream4(vbase + off + i * VSTRIDE) : 0u;
              }
            }
          }
        };

        // One slab.  A slab cut by the split bounds differs only in its
        // scores: rows outside the split score -inf (probability 0), and their
        // keys and values were loaded as zeros.
        auto compute = [&](int sl, const MFrag<DT, D, SL>& f) {
          const Pos q = pos(sl);

          // scores of each group: sc[g][i] = q_{4*grp+i} . k_{tb+16g+col}
          f32x4_t sc[L::NG];
  #pragma unroll
          for (int g = 0; g < L::NG; ++g) {
            sc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
            for (int st = 0; st < L::KS; ++st) {
              uint4 kb;
              if constexpr (DT == 1) {
                kb = f.k[g][st];
              } else if constexpr (DT == 2) {
                const uint4& w = f.k[g][st / 2];
                kb = (st & 1) ? fp8x8_to_bf16x8(w.z, w.w) : fp8x8_to_bf16x8(w.x, w.y);
              } else {
                kb = fp4x8_to_bf16x8(f.k4[g][st]);
              }
              sc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[st]),
                                                             __builtin_bit_cast(bf16x8_t, kb), sc[g],
                                                             0, 0, 0);
            }
            if constexpr (DT >= 2 && !kPacked) sc[g] *= f.ksc[g];
          }
          float alpha_h[G], nmc_h[G];
          bool moved = false;
          float* sp = s_p[wave];
          if constexpr (kPacked) {
            // The score tile of group g holds heads 0..3 in lanes 0..15 (rows
            // 4..15 of the A operand are empty); one lane shuffle per group
            // and register gathers the groups so that lane l holds token l of
            // the slab (group l / 16, column l % 16), register i head i.  The
            // K scale, split mask, exponentials, exp-sums, V scale and the
            // store for the value product then run once per token, every lane
            // busy, instead of once per (group, row); the per-head maxima
            // reduce over the whole wave.
            float X[4];
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              // row k of lanes takes row 0 of group k's tile
              float x = sc[0][i];
  #pragma unroll
              for (int g = 1; g < L::NG; ++g) {
                const float y = __shfl(sc[g][i], lane - 16 * g, kWave);
                x = grp == g ? y : x;
              }
              X[i] = x;
            }
            const int t = lane;                          // the lane's token in the slab
            const bool has_tok = L::NG == 4 || grp < 2;  // with two groups, lanes 32..63 hold none
            // K and V scales of token t
            const float ks = f.ksc[0], vs = f.vsc[0];
            bool valid = has_tok;
            if (!q.whole) valid = valid && q.tb + t >= t0 && q.tb + t < t1;
  #pragma unroll
            for (int i = 0; i < 4; ++i) X[i] = valid ? X[i] * ks : neg_inf();
  #pragma unroll
            for (int h = 0; h < G; ++h) {
              // the rows' maxima combined across the rows
              float r = row_max16(X[h]);
              r = fmaxf(r, __shfl_xor(r, 16, kWave));
              if constexpr (L::NG == 4) r = fmaxf(r, __shfl_xor(r, 32, kWave));
              const float mx = __builtin_bit_cast(
                  float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, r)));
              const float mn = fmaxf(m_h[h], mx);
              const float ms = mn != neg_inf() ? mn : 0.f;
              alpha_h[h] = fast_exp2((m_h[h] - ms) * c);
              nmc_h[h] = -ms * c;
              moved |= mn != m_h[h];
              m_h[h] = mn;
            }
            const int tb = t % KB;
            const int slot = (t - tb) + (KB / 4) * (tb & 3) + (tb >> 2);
  #pragma unroll
            for (int h = 0; h < G; ++h) {
              const float pv = fast_exp2(fmaf(X[h], c, nmc_h[h]));
              e_l[h] = fmaf(e_l[h], alpha_h[h], pv);
              if (has_tok) sp[h * SL + slot] = pv * vs;
            }
          } else {
            if (!q.whole) {  // wave-uniform branch
  #pragma unroll
              for (int g = 0; g < L::NG; ++g) {
                const int tk = q.tb + 16 * g + col;
                const bool kvalid = tk >= t0 && tk < t1;
  #pragma unroll
                for (int i = 0; i < 4; ++i) sc[g][i] = kvalid ? sc[g][i] : neg_inf();
              }
            }

            // slab maxima per head, then the running maxima (wave-uniform)
            float rm[4];
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              float x = sc[0][i];
  #pragma unroll
              for (int g = 1; g < L::NG; ++g) x = fmaxf(x, sc[g][i]);
              rm[i] = row_max16(x);
            }
  #pragma unroll
            for (int h = 0; h < G; ++h) {
              const float mx = lane_value(rm[h & 3], 16 * (h >> 2));
              const float mn = fmaxf(m_h[h], mx);
              const float ms = mn != neg_inf() ? mn : 0.f;
              alpha_h[h] = fast_exp2((m_h[h] - ms) * c);
              nmc_h[h] = -ms * c;
              moved |= mn != m_h[h];
              m_h[h] = mn;
            }

            // probabilities in the score layout (0 for rows scored -inf);
            // exp-sums per token column
            float pw[L::NG][4];
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int hi = (i < G) ? i : 0;
              float nmc = nmc_h[hi], al = alpha_h[hi];
              if constexpr (G > 4) {
                if (grp == 1) {
                  nmc = nmc_h[4 + i];
                  al = alpha_h[4 + i];
                }
              }
              float sum = 0.f;
  #pragma unroll
              for (int g = 0; g < L::NG; ++g) {
                pw[g][i] = fast_exp2(fmaf(sc[g][i], c, nmc));
                sum += pw[g][i];
              }
              e_l[i] = fmaf(e_l[i], al, sum);
            }

            // probabilities to the value-product operand layout (per-wave LDS);
            // over 8-bit pages each carries its token's V scale
            if (grp < HS) {
  #pragma unroll
              for (int g = 0; g < L::NG; ++g)
  #pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (4 * grp + i < G) {
                    const float pv = DT >= 2 ? pw[g][i] * f.vsc[g] : pw[g][i];
                    if constexpr (kDense) {
                      // head-major, each value block's tokens ordered by
                      // (token % 4, token / 4) so that a lane's operand is
                      // contiguous
                      const int t = 16 * g + col;
                      const int tb = t % KB;
                      sp[(4 * grp + i) * SL + (t - tb) + (KB / 4) * (tb & 3) + (tb >> 2)] = pv;
                    } else {
                      sp[(16 * g + col) * G + 4 * grp + i] = pv;
                    }
                  }
            }
          }

          if (wave_any(moved)) {  // scalar branch: skipped, not masked
            if constexpr (kDense) {
              // row 4*(lane/16) + i belongs to head (row % G)
              float al[4];
  #pragma unroll
              for (int i = 0; i < 4; ++i) {
                al[i] = alpha_h[i % G];
                if constexpr (G > 4) {
                  if (grp & 1) al[i] = alpha_h[4 + i];
                }
              }
  #pragma unroll
              for (int k = 0; k < 8; ++k)
  #pragma unroll
                for (int i = 0; i < 4; ++i) acc[0][k][i] *= al[i];
            } else {
  #pragma unroll
              for (int hs = 0; hs < HS; ++hs)
  #pragma unroll
                for (int k = 0; k < 8; ++k)
  #pragma unroll
                  for (int i = 0; i < 4; ++i)
                    if (4 * hs + i < G) acc[hs][k][i] *= alpha_h[4 * hs + i];
            }
          }

          if constexpr (kDense) {
            dense_values<DT, D, G, SL>(sp, f, acc[0]);
          } else {
          // value sums: acc[hs][k] += p[4hs + i][token] * v[token][dim k of this lane]
  #pragma unroll
          for (int j = 0; j < L::NI; ++j) {
            float pa[HS];
  #pragma unroll
            for (int hs = 0; hs < HS; ++hs) {
              pa[hs] = (4 * hs + quad < G) ? sp[(j * L::TPI + vrow) * G + 4 * hs + quad] : 0.f;
            }
            float vf[8];
            if constexpr (DT == 1) {
              const uint32_t w4[4] = {f.v[j].x, f.v[j].y, f.v[j].z, f.v[j].w};
  #pragma unroll
              for (int k = 0; k < 4; ++k) {
                vf[2 * k] = bf16_lo(w4[k]);
                vf[2 * k + 1] = bf16_hi(w4[k]);
              }
            } else if constexpr (DT == 2) {
              fp8x4_to_f32(f.v8[j].x, vf);
              fp8x4_to_f32(f.v8[j].y, vf + 4);
            } else {
              fp4x8_to_f32(f.v4[j], vf);
            }
  #pragma unroll
            for (int k = 0; k < 8; ++k) {
  #pragma unroll
              for (int hs = 0; hs < HS; ++hs)
                acc[hs][k] = __builtin_amdgcn_mfma_f32_4x4x1f32(pa[hs], vf[k], acc[hs][k], 0, 0, 0);
            }
          }
          }
        };

        constexpr int W = kMicroWaves;
        // Two slabs in flight while one is computed (three fragments taking
        // turns) wherever the registers hold them: 16-token slabs (with G = 8
        // only under the dense value product) and the plain instances'
        // 32-token 8-bit slabs with G <= 4; one where they do not: 4-bit 32-
        // and 64-token slabs, 8-bit 32-token slabs with G = 8, G = 8 at D = 64,
        // and the bf16 and 32-token 8-bit slabs of the fused instances (the
        // merge's code).
        constexpr bool kTwoInFlight =
            (G != 8 || kDense) &&
            (SL == 16 ? (DT != 1 || !kFused) : (DT == 2 && SL == 32 && G != 8 && !kFused));
        if constexpr (!kTwoInFlight) {
          MFrag<DT, D, SL> fa, fb;
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
        } else {
          // the three fragments take turns (no register copies, which would
          // have to wait for the loads in flight)
          MFrag<DT, D, SL> f0, f1, f2;
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
        }
        __syncthreads();  // the page list is rewritten by the next batch
      }
    }

    // ---- per-wave totals: exp-sums over token columns, values over token rows ----
    float we[G];
  #pragma unroll
    for (int h = 0; h < G; ++h) {
      float x = e_l[h & 3];
      x = x + dpp<kDppQuadXor1>(x);
      x = x + dpp<kDppQuadXor2>(x);
      x = x + dpp<kDppHalfMirror>(x);
      x = x + dpp<kDppRowMirror>(x);
      if constexpr (kPacked) {  // one token per lane: every row holds part of the sum
        we[h] = (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
      } else {
        we[h] = lane_value(x, 16 * (h >> 2));
      }
    }
    float accg[G][8];
    if constexpr (kDense) {
      // each head's high and low rows, summed over the lanes of a column below
  #pragma unroll
      for (int h = 0; h < G; ++h)
  #pragma unroll
        for (int k = 0; k < 8; ++k) {
          if constexpr (G == 2) {
            accg[h][k] = acc[0][k][h] + acc[0][k][h + 2];
          } else if constexpr (G == 4) {
            accg[h][k] = acc[0][k][h];
          } else {
            accg[h][k] = ((grp & 1) == (h >> 2)) ? acc[0][k][h & 3] : 0.f;
          }
        }
    } else {
  #pragma unroll
      for (int h = 0; h < G; ++h)
  #pragma unroll
        for (int k = 0; k < 8; ++k) accg[h][k] = acc[h >> 2][k][h & 3];
    }
  #pragma unroll
    for (int off = L::LPT; off < kWave; off <<= 1)
  #pragma unroll
      for (int h = 0; h < G; ++h)
  #pragma unroll
        for (int k = 0; k < 8; ++k) accg[h][k] += __shfl_xor(accg[h][k], off, kWave);

    finish_item<G, D, L::LPT, 8, kFused>(p, it, s_fin, m_h, we, accg, c);
  });
}

// Resident workgroups per CU (measured best for the grouped-query workload).
constexpr int kMfmaWorkgroupsPerCU = 2;

template <int DT, int D, int G, int SL>
hipError_t launch_one(const MicroParams& p, hipStream_t stream) {
  return launch_micro_step<D>(micro_mfma_kernel<DT, D, G, SL, false>,
                              micro_mfma_kernel<DT, D, G, SL, true>, kMfmaWorkgroupsPerCU, p, stream);
}

// bf16 pages: 16-token slabs.  fp8 pages: 32-token slabs (two score groups
// under one softmax update, 8 KiB of K + V like a bf16 slab) when the page
// size allows (G = 8: at D = 128 only); fp4 pages: 64-token slabs (four score
// groups, 8 KiB at D = 128), else 32 (G = 8: both at D = 128 only);
// otherwise 16-token slabs.  G = 8 over 16-token quantized slabs measured 9%
// (8-bit) and 33% (4-bit) slower on the grouped-query batch.
template <int DT, int D>
hipError_t dispatch_g(int G, const MicroParams& p, hipStream_t stream) {
  if constexpr (DT == 2) {
    if (p.P % 32 == 0 && G == 2) return launch_one<DT, D, 2, 32>(p, stream);
    if (p.P % 32 == 0 && G == 4) return launch_one<DT, D, 4, 32>(p, stream);
    if constexpr (D == 128)
      if (p.P % 32 == 0 && G == 8) return launch_one<DT, D, 8, 32>(p, stream);
  }
  if constexpr (DT == 3) {
    if (p.P % 64 == 0 && G == 2) return launch_one<DT, D, 2, 64>(p, stream);
    if (p.P % 64 == 0 && G == 4) return launch_one<DT, D, 4, 64>(p, stream);
    if constexpr (D == 128)
      if (p.P % 64 == 0 && G == 8) return launch_one<DT, D, 8, 64>(p, stream);
    if (p.P % 32 == 0 && G == 2) return launch_one<DT, D, 2, 32>(p, stream);
    if (p.P % 32 == 0 && G == 4) return launch_one<DT, D, 4, 32>(p, stream);
    if constexpr (D == 128)
      if (p.P % 32 == 0 && G == 8) return launch_one<DT, D, 8, 32>(p, stream);
  }
  switch (G) {
    case 2: return launch_one<DT, D, 2, 16>(p, stream);
    case 4: return launch_one<DT, D, 4, 16>(p, stream);
    case 8: return launch_one<DT, D, 8, 16>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// 8-bit pages: micro_mfma_kernel<2, ...> for G in {2, 4, 8}, compiled in a
// translation unit of its own (micro_attention_mfma_fp8.hip, built with NaNs
// ruled out and IEEE mode off so that its DPP max steps fold).
hipError_t launch_micro_mfma_fp8(int D, int G, const MicroParams& p, hipStream_t stream);
// 4-bit pages: micro_mfma_kernel<3, ...>, likewise in a translation unit of its
// own (micro_attention_mfma_fp4.hip) with the same flags.
hipError_t launch_micro_mfma_fp4(int D, int G, const MicroParams& p, hipStream_t stream);

}  // namespace da
