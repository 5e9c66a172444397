/*
 * da.h -- C ABI of the split-KV decode attention library (libda.so, gfx950).
 *
 * The library computes decode-phase attention of one query token per
 * (request, query head) over a paged KV cache in two steps:
 *
 *   da_micro_attention  MicroAttention per (request, query head, split):
 *                         m_j  = max_i s_i
 *                         e_j  = sum_i exp(s_i - m_j)
 *                         MA_j = sum_i exp(s_i - m_j) * v_i
 *                       with s_i = scale * (q . k_i).
 *                       (Infinite-LLM page, section 方法细节, the MicroAttention
 *                       equations of the equivalent transform.)
 *   da_merge            aggregation of the b partials of each (request, head):
 *                         m_g = max_j m_j
 *                         e_g = sum_j e_j * exp(m_j - m_g)
 *                         out = sum_j MA_j * exp(m_j - m_g) / e_g
 *                       (Infinite-LLM page, section 方法细节, the aggregation
 *                       equations.)
 *
 * Whole KV pages can be skipped with a block mask (LServe blog page, section
 * 2.1.1: only the selected blocks are loaded and computed).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array argument is DEVICE memory owned by the caller.  The library
 *   keeps no pointer after a call returns and allocates nothing: scratch
 *   space comes in as a caller-provided workspace.
 * - Calls only enqueue work on `stream` (0 = the null stream) and return; the
 *   caller synchronises.  Calls are re-entrant and may run concurrently on
 *   different streams when their output buffers do not overlap.
 * - A call that returns anything but DA_OK has enqueued nothing (argument
 *   errors are found on the host before any launch), except DA_ERR_HIP, which
 *   reports a failed launch.  da_last_error() then describes the failure.
 * - Array CONTENTS are trusted: block-table entries must index pages of the
 *   pool and values must be finite on every token that a split reads.  Slots
 *   that no split reads (tail of a partial last page, masked pages, pages the
 *   table does not name) are never loaded and may hold anything.
 *   da_check_inputs() validates the contents on the device.
 */
#ifndef DA_H
#define DA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum da_status {
  DA_OK = 0,
  DA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or shape     */
  DA_ERR_UNSUPPORTED = 2, /* valid but not built: D, P, dtype or group size  */
  DA_ERR_HIP = 3          /* a HIP runtime call or kernel launch failed      */
} da_status;

typedef enum da_dtype {
  DA_F32 = 0,     /* IEEE binary32                                     */
  DA_BF16 = 1,    /* bfloat16: the upper 16 bits of an IEEE binary32  */
  DA_FP8_E4M3 = 2, /* 8-bit pages: OCP FP8 E4M3 codes with one fp32    */
                   /* scale per (page, KV head, slot) row; q is bf16.  */
                   /* Used by the *_fp8 entry points only.             */
  DA_FP4_E2M1 = 3  /* 4-bit pages: OCP FP4 E2M1 codes, two per byte,   */
                   /* with one fp32 scale per row; q is bf16.  Used by */
                   /* the *_fp4 entry points only.                     */
} da_dtype;

/* Order of the dimensions of the K / V pools.  Page-major: [NP, Hkv, P, D]
 * (a physical page holds every KV head).  Head-major: [Hkv, NP, P, D] (one
 * KV head's pages form one contiguous run: the per-head view
 * K:[num_pages, page_size, head_dim] of the LServe blog page, section 3.1.2,
 * stacked over heads); the fp8 scale arrays follow the same order. */
typedef enum da_pool_layout {
  DA_POOL_PAGE_MAJOR = 0,
  DA_POOL_HEAD_MAJOR = 1
} da_pool_layout;

/* Problem shape.  Notation: S requests, Hq query heads, Hkv KV heads
 * (G = Hq / Hkv query heads share one KV head: query head h reads KV head
 * h / G), D head dimension, P tokens per page, NP pages in the pool. */
typedef struct da_shape {
  int32_t S;
  int32_t Hq;
  int32_t Hkv;
  int32_t D;               /* 64 or 128                                        */
  int32_t P;               /* 16, 32, 64, 128 or 256                           */
  int32_t max_pages;       /* row length of block_table and block_mask;       */
                           /* (max_pages + 1) * P must fit in int32            */
  int32_t max_splits;      /* b: splits per (request[, KV head]), >= 1          */
  int32_t bounds_per_head; /* 0: split_bounds is [S, 1, b+1]; 1: [S, Hkv, b+1]  */
  int32_t dtype;           /* da_dtype of q, k_pages and v_pages               */
  float scale;             /* score scale, > 0 and finite (usually 1/sqrt(D))  */
  int64_t NP;              /* pages in k_pages / v_pages, >= 1                 */
  int32_t chunks;          /* 0: library choice; 1..64: each split is cut into  */
                           /* this many page ranges, processed independently   */
                           /* and folded back (needs a workspace)              */
  int32_t schedule;        /* 0: library choice; 1: one workgroup per item;     */
                           /* 2: persistent workgroups claiming items from     */
                           /* work queues in the workspace                     */
  int32_t pool_layout;     /* da_pool_layout of the K / V pools (and fp8 scale  */
                           /* arrays); read by every call that takes them      */
  int32_t fuse;            /* read by da_attention* only: 0 library choice;    */
                           /* 1 one launch (each group merged by the item that */
                           /* completes it); 2 two launches (partials into the */
                           /* workspace, then the merge kernel)                */
} da_shape;

/*
 * MicroAttention partials for every (request s, query head h, split j).
 *
 * Inputs (device, caller-owned):
 *   q            [S, Hq, D] of sh->dtype, 16-byte aligned.
 *   k_pages      [NP, Hkv, P, D] of sh->dtype, 16-byte aligned: the key of
 *                logical token t of request s for KV head g is
 *                k_pages[block_table[s, t / P], g, t % P, :]; with
 *                sh->pool_layout = DA_POOL_HEAD_MAJOR the pool is
 *                [Hkv, NP, P, D] and the key is k_pages[g, block_table[s, t / P],
 *                t % P, :] (every call that takes pools reads this field, and
 *                8-bit scale arrays [NP, Hkv, P] become [Hkv, NP, P]).
 *   v_pages      same layout as k_pages, for values.
 *   block_table  [S, max_pages] int32: logical page -> physical page.  Only
 *                entries of pages that hold tokens of some split are read.
 *   seq_lens     [S] int32: context length L_s, 0 <= L_s <= max_pages * P.
 *   split_bounds [S, 1, b+1] or [S, Hkv, b+1] int32 token offsets.  Split j
 *                of request s (and KV head g when bounds are per head) is the
 *                token range [sb_j, sb_{j+1}) intersected with [0, L_s).  The
 *                usual choice is 0 = sb_0 <= ... <= sb_b = L_s, padded by
 *                repeating L_s, but any values are accepted: an inverted or
 *                out-of-range split is empty.  Ranges from different calls may
 *                cover different parts of a request; their partials merge.
 *   block_mask   NULL, or [S, Hkv, max_pages] uint8: page lp of request s is
 *                skipped for KV head g (and its G query heads) when
 *                block_mask[s, g, lp] == 0.
 * Outputs (device, caller-owned, fully written):
 *   MA           [S, Hq, b, D] float32, 16-byte aligned.
 *   m, e         [S, Hq, b] float32.  m is in the natural-log domain of the
 *                scaled score.  An empty split (no kept token) is written as
 *                MA = 0, m = -inf, e = 0.
 * Workspace (device, caller-owned, 16-byte aligned, contents irrelevant):
 *   da_micro_attention_workspace_size() bytes.  It holds work-queue
 *   counters (512 bytes, reset on `stream` by the call itself) used when
 *   the grid of (request, KV head, split) items is far larger than the GPU
 *   can hold at once, and the partials of page-range chunks that every split is cut
 *   into and folded back afterwards: with sh->chunks == 0, when there are
 *   fewer items than the GPU runs at once, or when splits are long (4 MiB
 *   of K and V or more) and cutting them balances the launch.
 *   With sh->chunks == 0 and a NULL or smaller workspace the call runs with
 *   one workgroup per unchunked item (same results, possibly slower); with
 *   sh->chunks > 1 a missing workspace is DA_ERR_INVALID_ARG.  Concurrent
 *   calls must not share a workspace.
 * Errors: DA_ERR_INVALID_ARG, DA_ERR_UNSUPPORTED (D, P, dtype or G = Hq/Hkv
 * outside the built set {1, 2, 4, 8}), DA_ERR_HIP.
 */
da_status da_micro_attention(const da_shape* sh, const void* q, const void* k_pages,
                             const void* v_pages, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* split_bounds,
                             const uint8_t* block_mask, float* MA, float* m, float* e,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes da_micro_attention uses for this shape (0 if it runs
 * unchunked).  Host-only; writes *bytes. */
da_status da_micro_attention_workspace_size(const da_shape* sh, size_t* bytes);

/*
 * MicroAttention over 8-bit KV pages (LServe blog page, section 3.2.1: the
 * retrieval-head cache is stored with configurable 2-8 bit quantization).
 * Same partials, splits, mask, workspace and errors as da_micro_attention,
 * with sh->dtype = DA_FP8_E4M3 and:
 *   q            [S, Hq, D] bfloat16, 16-byte aligned.
 *   k_codes      [NP, Hkv, P, D] uint8 OCP FP8 E4M3 codes, 16-byte aligned;
 *                the key of a token is value(code) * k_scales[page, g, slot]
 *                (per-row scales as written by da_quantize_rows).
 *   k_scales     [NP, Hkv, P] float32, 4-byte aligned.
 *   v_codes, v_scales  likewise for values.
 * Scores, softmax and value sums are computed in fp32 from the exact code
 * values; slots outside every split are never read.  Supported: D 64 or 128,
 * G in {1, 2, 4, 8}.  da_micro_attention_workspace_size with the same shape
 * gives the workspace size.
 */
da_status da_micro_attention_fp8(const da_shape* sh, const void* q, const uint8_t* k_codes,
                                 const float* k_scales, const uint8_t* v_codes,
                                 const float* v_scales, const int32_t* block_table,
                                 const int32_t* seq_lens, const int32_t* split_bounds,
                                 const uint8_t* block_mask, float* MA, float* m, float* e,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * 8-bit quantization of rows (the write side of 8-bit KV pages): for each of
 * `rows` rows of D elements of x (dtype DA_F32 or DA_BF16, [rows, D],
 * 16-byte aligned), s = amax / 448 (amax = the largest |x| of the row, fp32
 * division) and code = the OCP FP8 E4M3 value nearest to x / s (fp32
 * division, clamped to [-448, 448], ties to even, sign kept when the
 * magnitude rounds to zero); an all-zero row gets s = 0 and codes 0.
 * codes [rows, D] uint8 (8-byte aligned), scales [rows] float32.  A K or V
 * pool [NP, Hkv, P, D] is rows = NP * Hkv * P.  Supported: D 64 or 128.
 */
da_status da_quantize_rows(int32_t dtype, int64_t rows, int32_t D, const void* x,
                           uint8_t* codes, float* scales, hipStream_t stream);

/*
 * Decode-time append into 8-bit pages: the write of da_append_kv (token
 * t = seq_lens[s] of every request with 0 <= t < max_pages * P, through the
 * block table; seq_lens is not advanced) for pools of OCP FP8 E4M3 codes
 * with per-row scales.  The new rows k_new, v_new ([S, Hkv, D] of sh->dtype,
 * DA_F32 or DA_BF16, 16-byte aligned) are quantized exactly as
 * da_quantize_rows does, and their codes and scales are written to
 * k_codes / v_codes ([NP, Hkv, P, D] uint8, 8-byte aligned) and k_scales /
 * v_scales ([NP, Hkv, P] float32) at the token's slot.  If stats is not
 * NULL ([Hkv, NP, P / logical, 2, D] of sh->dtype, as for da_page_stats),
 * the statistics of the receiving logical page are kept current from the
 * full-precision key row exactly as da_append_kv does (select_heads and
 * logical as there), so page selection keeps working on 8-bit pools.  Reads
 * sh->S, Hkv, D, P, NP, max_pages, dtype.  Supported: D 64 or 128.  As for
 * da_append_kv, a block-table entry outside [0, NP) for the receiving page
 * writes nothing for that request.
 */
da_status da_append_kv_fp8(const da_shape* sh, const void* k_new, const void* v_new,
                           const int32_t* block_table, const int32_t* seq_lens, uint8_t* k_codes,
                           float* k_scales, uint8_t* v_codes, float* v_scales, int32_t logical,
                           const uint8_t* select_heads, void* stats, hipStream_t stream);

/*
 * 4-bit KV pages (LServe blog page, section 3.2.1: the streaming-head cache
 * is stored in 4 bits, the retrieval-head cache with 2-8 bits).  Format:
 * OCP FP4 E2M1 codes (1 sign bit, 2 exponent bits with bias 1, 1 mantissa
 * bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN), two per
 * byte, element 2i of a row in the low nibble of byte i; one fp32 scale per
 * row, s = amax / 6 (fp32 division), code = the E2M1 value nearest to x / s
 * (fp32 division; |x / s| clamped to 6; ties to the code with mantissa bit
 * 0; the sign kept when the magnitude rounds to zero); an all-zero row has
 * s = 0 and codes 0.  A key or value stands for value(code) * s.
 *
 * da_quantize_rows_fp4: as da_quantize_rows with codes [rows, D / 2] uint8
 *   (4-byte aligned) in this format.
 * da_append_kv_fp4: as da_append_kv_fp8, writing 4-bit code rows of D / 2
 *   bytes (pools [NP, Hkv, P, D / 2], 4-byte aligned) and their scales.
 * da_micro_attention_fp4, da_attention_fp4: as the _fp8 entry points with
 *   sh->dtype = DA_FP4_E2M1 and code pools [NP, Hkv, P, D / 2] uint8
 *   (16-byte aligned; head-major [Hkv, NP, P, D / 2] with
 *   DA_POOL_HEAD_MAJOR).  Supported: D 64 or 128 (D = 64 with one query
 *   head per KV head needs P >= 32), G in {1, 2, 4, 8}; workspace sizes
 *   from the same queries as the other pages.
 */
da_status da_quantize_rows_fp4(int32_t dtype, int64_t rows, int32_t D, const void* x,
                               uint8_t* codes, float* scales, hipStream_t stream);
da_status da_append_kv_fp4(const da_shape* sh, const void* k_new, const void* v_new,
                           const int32_t* block_table, const int32_t* seq_lens, uint8_t* k_codes,
                           float* k_scales, uint8_t* v_codes, float* v_scales, int32_t logical,
                           const uint8_t* select_heads, void* stats, hipStream_t stream);
da_status da_micro_attention_fp4(const da_shape* sh, const void* q, const uint8_t* k_codes,
                                 const float* k_scales, const uint8_t* v_codes,
                                 const float* v_scales, const int32_t* block_table,
                                 const int32_t* seq_lens, const int32_t* split_bounds,
                                 const uint8_t* block_mask, float* MA, float* m, float* e,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);
da_status da_attention_fp4(const da_shape* sh, const void* q, const uint8_t* k_codes,
                           const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                           const int32_t* block_table, const int32_t* seq_lens,
                           const int32_t* split_bounds, const uint8_t* block_mask, float* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Aggregate b partials per (request, query head) into attention output.
 *
 *   MA [S, Hq, b, D], m [S, Hq, b], e [S, Hq, b] float32 as written by
 *   da_micro_attention (or gathered from several calls: the merge accepts any
 *   partials that follow the same convention, in any order).
 *   out [S, Hq, D] float32.  A (request, head) whose partials are all empty
 *   gets out = 0.
 * Only sh->S, sh->Hq, sh->D and sh->max_splits (= b) are read.
 * Errors: DA_ERR_INVALID_ARG, DA_ERR_HIP.
 */
da_status da_merge(const da_shape* sh, const float* MA, const float* m, const float* e,
                   float* out, hipStream_t stream);

/*
 * One decode step in a single launch: the MicroAttention partials of every
 * split and their aggregation into the attention output (Infinite-LLM page,
 * section 方法细节: local MicroAttention per sub-block, then the aggregation
 * equations), i.e. da_micro_attention followed by da_merge, with the merge
 * done by the work item that completes the last partial of each (request,
 * KV head) instead of by a second kernel.  sh->fuse picks the form: 1 that
 * one launch; 2 two launches (the partials of every piece into the
 * workspace, then the merge kernel over them); 0 the library's choice per
 * shape: one launch when the grid is one round of workgroups, two launches
 * otherwise (the shapes where each was measured faster); also two when the
 * one-launch kernel instance would spill registers.  Either form gives the
 * same result within fp32 rounding.
 *
 *   Inputs as for da_micro_attention (da_attention_fp8: as for
 *   da_micro_attention_fp8).
 *   out        [S, Hq, D] float32, caller-owned, fully written: the merge of
 *              the b splits (all-empty -> 0), within fp32 rounding of
 *              da_micro_attention + da_merge on the same inputs.
 *   workspace  device, caller-owned, 16-byte aligned, at least
 *              da_attention_workspace_size() bytes.  Its first counter_bytes
 *              (as returned there) hold one counter per (request, KV head)
 *              and MUST BE ZERO before the first call (zero-fill the buffer
 *              once when it is allocated); every call that completes leaves
 *              them zero, so later calls need no clearing.  Clear them again
 *              after using the buffer for anything else, or before a call
 *              whose S * Hkv exceeds every earlier one (the new counters
 *              then cover bytes that held partials).  The rest holds the
 *              partials and the work-queue counters.  Concurrent calls must not
 *              share a workspace.  A workspace too small is
 *              DA_ERR_INVALID_ARG (with sh->chunks == 0 the call first falls
 *              back to unchunked splits if those fit).
 * Every call only enqueues kernels on `stream` (no allocation, no host
 * synchronisation, no memset node), so a step can be captured in a HIP
 * graph and replayed.
 * Errors: as da_micro_attention.
 */
da_status da_attention(const da_shape* sh, const void* q, const void* k_pages, const void* v_pages,
                       const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* split_bounds, const uint8_t* block_mask, float* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

da_status da_attention_fp8(const da_shape* sh, const void* q, const uint8_t* k_codes,
                           const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                           const int32_t* block_table, const int32_t* seq_lens,
                           const int32_t* split_bounds, const uint8_t* block_mask, float* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of da_attention / da_attention_fp8 for this shape, and
 * (counter_bytes, nullable) how many of its first bytes are the counters
 * that must start at zero.  Host-only. */
da_status da_attention_workspace_size(const da_shape* sh, size_t* bytes, size_t* counter_bytes);

/*
 * Fold b partials per (request, query head) into ONE partial triple and write
 * it into slot `out_slot` of a gather buffer: the aggregation equations of
 * the Infinite-LLM page (section 方法细节) without the final division,
 *   m'  = max_j m_j
 *   e'  = sum_j e_j * exp(m_j - m')
 *   MA' = sum_j MA_j * exp(m_j - m')
 * which is again the MicroAttention triple of the union of the partials'
 * token sets, so folded triples merge like any others.  This is an
 * instance's local step in distributed decoding (LoongServe page, section
 * 4.2, single- and multi-master decoding: instances compute local attention
 * and send results to the master): each instance folds its own splits, the
 * triples are gathered into one buffer, and the master calls da_merge on it
 * with max_splits = out_splits.
 *
 *   MA [S, Hq, b, D], m [S, Hq, b], e [S, Hq, b] float32 as for da_merge
 *   (b = sh->max_splits).
 *   MA_out [S, Hq, out_splits, D], m_out and e_out [S, Hq, out_splits]
 *   float32, caller-owned; only slot out_slot of each (request, head) is
 *   written, every other slot is left as it is.  A (request, head) whose
 *   partials are all empty gets (MA', m', e') = (0, -inf, 0).
 * The outputs must not overlap the inputs.  Reads sh->S, Hq, D and
 * max_splits only.
 * Errors: DA_ERR_INVALID_ARG (NULL or misaligned pointer, sizes < 1,
 * out_splits < 1, out_slot outside [0, out_splits)), DA_ERR_HIP.
 */
da_status da_merge_partials(const da_shape* sh, const float* MA, const float* m, const float* e,
                            int32_t out_splits, int32_t out_slot, float* MA_out, float* m_out,
                            float* e_out, hipStream_t stream);

/*
 * Device-side validation of the array contents that da_micro_attention
 * trusts: 0 <= seq_lens[s] <= max_pages * P for every request, and
 * 0 <= block_table[s, lp] < NP for every logical page lp < ceil(L_s / P)
 * (stricter than needed: it also covers pages that no split reads or the
 * mask skips).  Adds the number of violations found to err[0] (device int32,
 * caller-owned; set it to 0 first).  Reads sh->S, P, max_pages and NP only.
 */
da_status da_check_inputs(const da_shape* sh, const int32_t* block_table,
                          const int32_t* seq_lens, int32_t* err, hipStream_t stream);

/*
 * Hierarchical page selection for retrieval heads (LServe blog page, section
 * 2.2.2 "解码阶段创新": a physical page of P tokens holds logical pages of
 * `logical` tokens, each with per-dimension key statistics k_max / k_min,
 * and the important physical pages are picked from the query; section 3.1.2
 * "动态稀疏的层次化选择": statistics per logical page, a score per physical
 * page as the maximum over its logical pages, the top-K pages kept).  The
 * result is the block mask da_micro_attention consumes.
 *
 * Supported: dtype F32 or BF16 (q, K and the statistics share it), D 64 or
 * 128, G = Hq / Hkv in {1, 2, 4, 8}, logical in {8, 16, 32, 64} with
 * P / logical a power of two no larger than 256; da_select_pages also needs
 * max_pages <= 65536.  Anything else returns DA_ERR_UNSUPPORTED.  The calls
 * read sh->S, Hq, Hkv, D, P, NP, max_pages and dtype only.  select_heads is
 * a device uint8 [Hkv] array of retrieval-head flags, nullable = every head.
 *
 * da_page_stats: stats [Hkv, NP, P / logical, 2, D] (dtype, 16-byte
 *   aligned, caller-owned; head-major, so one KV head's statistics are one
 *   contiguous run): for every physical page that block_table names
 *   below ceil(L_s / P), and every KV head and logical sub-page, index 0 =
 *   the per-dimension maximum and index 1 = the per-dimension minimum of the
 *   keys of the sub-page's tokens below L_s (exact: the stored values
 *   themselves).  A sub-page with no token below L_s gets zeros.  Pages no
 *   table row names, and KV heads whose select_heads entry is 0, are not
 *   written.  k_pages as for da_micro_attention.  A physical page named by
 *   two table rows with different token counts on it gets either row's
 *   statistics.
 *
 * da_page_scores: scores [S, Hkv, max_pages] fp32 (4-byte aligned): for
 *   page lp < ceil(L_s / P) of request s and KV head kvh, the maximum over
 *   the group's query heads h (h / G == kvh) and over the logical sub-pages
 *   holding a token below L_s of the bound
 *       sum_d max(q_h[d] * kmax[d], q_h[d] * kmin[d])   (>= q_h . k for
 *   every key k of the sub-page), accumulated in fp32; -inf for pages at or
 *   beyond ceil(L_s / P), and for every page of a KV head whose entry in
 *   select_heads is 0.  The
 *   scores are raw bounds: no attention scale (it does not change the order).
 *
 * da_select_pages: block_mask [S, Hkv, max_pages] uint8 (caller-owned,
 *   every entry written): for a KV head with select_heads[kvh] != 0 (or
 *   select_heads NULL) the first keep_first and the last keep_last pages
 *   below ceil(L_s / P) are 1, and of the pages between them the `budget`
 *   with the highest score are 1 (equal scores: lower page index first;
 *   -0.0 equals 0.0); a KV head with select_heads[kvh] == 0 keeps every page
 *   below ceil(L_s / P).  Pages from ceil(L_s / P) up to
 *   ceil((L_s + horizon) / P) (at most max_pages) are 1 for every head: a
 *   selection reused while `horizon` more tokens are appended (section
 *   2.2.2, reusable page selector: select at the start of a chunk of decode
 *   steps, reuse inside it) then still covers the pages those tokens open.
 *   Pages beyond are 0.  budget, keep_first, keep_last and horizon must be
 *   >= 0.  Scores must not be NaN.
 */
da_status da_page_stats(const da_shape* sh, const void* k_pages, const int32_t* block_table,
                        const int32_t* seq_lens, int32_t logical, const uint8_t* select_heads,
                        void* stats, hipStream_t stream);
da_status da_page_scores(const da_shape* sh, const void* q, const void* stats,
                         const int32_t* block_table, const int32_t* seq_lens, int32_t logical,
                         const uint8_t* select_heads, float* scores, hipStream_t stream);
da_status da_select_pages(const da_shape* sh, const float* scores, const int32_t* seq_lens,
                          int32_t budget, int32_t keep_first, int32_t keep_last, int32_t horizon,
                          const uint8_t* select_heads, uint8_t* block_mask, hipStream_t stream);

/*
 * Decode-time KV append (the cache write of one decode step).  For every
 * request s with 0 <= t = seq_lens[s] < max_pages * P and every KV head kvh,
 * the key row k_new[s, kvh, :] and value row v_new[s, kvh, :] ([S, Hkv, D],
 * dtype, 16-byte aligned) are written to k_pages / v_pages at page
 * block_table[s, t / P], slot t % P (the caller assigns that table entry
 * before the call).  Requests with t outside that range are skipped.  The
 * call does not change seq_lens: the caller advances it by one afterwards.
 *
 * If stats is not NULL ([Hkv, NP, P / logical, 2, D] as for da_page_stats),
 * the statistics of the logical page receiving the token are kept current at
 * write time (LServe blog page, section 3.1.2: statistics are computed when
 * the cache is written): for a KV head whose select_heads entry is not 0 (or
 * select_heads NULL), the first token of a logical page sets kmax = kmin =
 * the key, a later one folds in with max / min; the result equals
 * da_page_stats on the new contents at length t + 1.  logical is read only
 * when stats is not NULL.
 *
 * Reads sh->S, Hkv, D, P, NP, max_pages, dtype.  Supported: dtype F32 or
 * BF16, D 64 or 128 (statistics: as for da_page_stats).  Two requests must
 * not append into the same physical page in one call.  The block-table entry
 * of the receiving page (logical page t / P, which da_check_inputs does not
 * cover when t is a multiple of P) is checked on the device: an entry outside
 * [0, NP) writes nothing for that request.
 */
da_status da_append_kv(const da_shape* sh, const void* k_new, const void* v_new,
                       const int32_t* block_table, const int32_t* seq_lens, void* k_pages,
                       void* v_pages, int32_t logical, const uint8_t* select_heads, void* stats,
                       hipStream_t stream);

/*
 * Split bounds over the kept pages, computed on the device (work planning
 * for a mask that is reused across decode steps, so no host round trip is
 * needed).  For request s let E = min(seq_lens[s] + horizon, max_pages * P)
 * and consider pages below ceil(E / P); for KV head kvh let kept[0] < ... <
 * kept[K-1] be those with block_mask[s, kvh, page] != 0 (every page when
 * block_mask is NULL).  With b = sh->max_splits, split_bounds[s, kvh, :]
 * ([S, Hkv, b + 1] int32, the per-head layout of da_micro_attention) gets
 *     bound[0] = 0, bound[b] = E,
 *     bound[j] = P * kept[floor(j K / b)]   (0 < j < b; E when K = 0),
 * so every split holds floor(K / b) or ceil(K / b) kept pages (the
 * Infinite-LLM page's sub-blocks, balanced over the pages a mask keeps).
 * Reads sh->S, Hkv, P, max_pages, max_splits.  horizon must be >= 0.
 */
da_status da_split_bounds(const da_shape* sh, const uint8_t* block_mask, const int32_t* seq_lens,
                          int32_t horizon, int32_t* split_bounds, hipStream_t stream);

/*
 * The decode step of da_attention for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same inputs, output, forms (sh->fuse) and
 * results as da_attention (bf16 / fp32 pools), with no workspace argument:
 * the counters, work queue and partials live in a device array the library
 * holds for the life of the process, DA_NOALLOC_SCRATCH_BYTES (32 MiB) per
 * GPU, enough for every workload of the configurations C1-C5.  The call
 * allocates nothing and frees nothing; it clears the counters itself (a fill
 * kernel on `stream`) before the step.  A shape whose step needs more than
 * the array (da_attention_workspace_size, unchunked if the library's chunking
 * does not fit) is DA_ERR_INVALID_ARG before any launch.
 * The array is shared by every call on the same GPU and keeps the last
 * call's contents: calls that may overlap on one GPU (different streams
 * without ordering between them) race on it and must not be issued.
 * Errors: as da_attention; DA_ERR_HIP also when the array's device address
 * cannot be obtained.
 */
#define DA_NOALLOC_SCRATCH_BYTES (32u << 20)
da_status da_attention_noalloc(const da_shape* sh, const void* q, const void* k_pages,
                               const void* v_pages, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* split_bounds,
                               const uint8_t* block_mask, float* out, hipStream_t stream);

/* Message for the status of the calling thread's most recent da_* call that
 * returns a da_status: empty when that call returned DA_OK (every such entry
 * point clears it first).  Thread-local; never NULL. */
const char* da_last_error(void);

/*
 * Measurement helper, not part of the attention path: reads `bytes` bytes of
 * device memory at `src` (16-byte aligned, bytes a multiple of 16) with
 * coalesced 16-byte loads and writes one 32-bit word per workgroup into
 * `sink` (device, >= da_stream_read_sink_words() words) so the reads cannot be
 * elided.  Gives the achievable HBM read rate on this device.
 */
da_status da_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
size_t da_stream_read_sink_words(void);

#ifdef __cplusplus
}
#endif

#endif /* DA_H */
