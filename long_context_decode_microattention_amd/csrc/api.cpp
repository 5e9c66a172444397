// Public C ABI of libda.so (include/da.h): argument validation on the host,
// status codes with a thread-local message, and dispatch to the kernels.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <hip/hip_runtime.h>

#include <climits>
#include <mutex>
#include <string>

#include "da.h"
#include "launch.h"

namespace {

constexpr int kMaxChunks = 64;
constexpr int kAutoMaxChunks = 16;
constexpr long long kBalanceItemBytes = 4LL << 20;  // splits this large are cut for balance

thread_local std::string g_last_error;

da_status fail(da_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// Shape checks shared by the entry points that read the paged cache.  The
// quantized page types (8- and 4-bit) are accepted only where quant is true
// (their own entry points and the workspace queries).
da_status check_shape(const da_shape* sh, bool quant = false) {
  if (sh == nullptr) return fail(DA_ERR_INVALID_ARG, "shape is NULL");
  if (sh->S < 1 || sh->Hq < 1 || sh->Hkv < 1 || sh->D < 1 || sh->P < 1 || sh->max_pages < 1 ||
      sh->max_splits < 1 || sh->NP < 1)
    return fail(DA_ERR_INVALID_ARG,
                "sizes must be >= 1 (S=%d Hq=%d Hkv=%d D=%d P=%d max_pages=%d max_splits=%d NP=%lld)",
                sh->S, sh->Hq, sh->Hkv, sh->D, sh->P, sh->max_pages, sh->max_splits,
                (long long)sh->NP);
  if (sh->Hq % sh->Hkv != 0)
    return fail(DA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", sh->Hq, sh->Hkv);
  if (sh->bounds_per_head != 0 && sh->bounds_per_head != 1)
    return fail(DA_ERR_INVALID_ARG, "bounds_per_head must be 0 or 1 (got %d)", sh->bounds_per_head);
  const bool quantized = sh->dtype == DA_FP8_E4M3 || sh->dtype == DA_FP4_E2M1;
  if (sh->dtype != DA_F32 && sh->dtype != DA_BF16 && !(quant && quantized))
    return fail(DA_ERR_INVALID_ARG, "dtype %d is not a da_dtype%s", sh->dtype,
                quantized ? " for this entry point (quantized pages: da_micro_attention_fp8 / _fp4)" : "");
  if (!(sh->scale > 0.f) || !isfinite(sh->scale))
    return fail(DA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if ((long long)sh->max_pages * sh->P > (long long)INT_MAX - sh->P)
    return fail(DA_ERR_INVALID_ARG, "max_pages * P + P exceeds the int32 token range");
  // stepwise: each partial product is checked before it is multiplied again
  if ((long long)sh->S * sh->Hkv > INT_MAX ||
      (long long)sh->S * sh->Hkv * sh->max_splits > INT_MAX)
    return fail(DA_ERR_INVALID_ARG, "S * Hkv * max_splits exceeds the launch range");
  if (sh->NP > (long long)INT_MAX + 1)
    return fail(DA_ERR_INVALID_ARG, "NP exceeds the int32 block-table range");
  if (sh->schedule < 0 || sh->schedule > 2)
    return fail(DA_ERR_INVALID_ARG, "schedule must be 0, 1 or 2 (got %d)", sh->schedule);
  if (sh->pool_layout != DA_POOL_PAGE_MAJOR && sh->pool_layout != DA_POOL_HEAD_MAJOR)
    return fail(DA_ERR_INVALID_ARG, "pool_layout must be DA_POOL_PAGE_MAJOR or DA_POOL_HEAD_MAJOR (got %d)",
                sh->pool_layout);
  if (sh->chunks < 0 || sh->chunks > kMaxChunks)
    return fail(DA_ERR_INVALID_ARG, "chunks must be 0 (library choice) or 1..%d (got %d)",
                kMaxChunks, sh->chunks);
  if (sh->fuse < 0 || sh->fuse > 2)
    return fail(DA_ERR_INVALID_ARG, "fuse must be 0, 1 or 2 (got %d)", sh->fuse);
  return DA_OK;
}

// Chunks per split.  A launch wants enough workgroups that every compute
// unit holds several and the dispatcher can even out unequal items (dense vs
// masked heads, ragged lengths); below that target, splits are cut into page
// ranges, at most as many as a split of an evenly divided max-length request
// has pages.
// Compute units of the current device (256 on MI355X when the query fails).
long long device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return 256;
  return cus;
}

// Chunks per split when the caller leaves the choice to the library.  A
// chunked launch adds the combine kernel (5-9 us of a replayed step), so
// splits are cut for two reasons only:
//  - to fill the device: fewer work units than it runs at once leave compute
//    units idle.  One workgroup of the vector kernel per CU already draws
//    most of the bandwidth; the GQA kernel wants two (measured on single
//    requests: 16 x 4K tokens over 256 splits runs best uncut, 8K tokens of
//    GQA 32/8 over 32 splits best in 16 chunks);
//  - to balance long items: splits of several MiB whose kept lengths differ
//    (block-sparse heads beside dense ones) finish together when cut into
//    more, shorter units (the chunk counts measured best on the 512K GQA
//    batch).
int resolve_chunks(const da_shape* sh) {
  if (sh->chunks > 0) return sh->chunks;
  const int G = sh->Hq / sh->Hkv;
  const long long items = (long long)sh->S * sh->Hkv * sh->max_splits;
  const long long pages_per_split = sh->max_pages / sh->max_splits;  // typical split size
  const long long row = sh->dtype == DA_F32    ? 4LL * sh->D
                        : sh->dtype == DA_BF16   ? 2LL * sh->D
                        : sh->dtype == DA_FP8_E4M3 ? sh->D + 4LL
                                                   : sh->D / 2 + 4LL;  // codes plus the row scale
  const long long item_bytes = pages_per_split * sh->P * 2 * row;  // K and V of a typical split
  const long long fill = device_cus() * (da::micro_mfma_supported(sh->dtype, sh->D, G) ? 2 : 1);
  long long c = (fill + items - 1) / items;
  if (item_bytes >= kBalanceItemBytes) {
    const long long target = da::micro_target_items(sh->dtype, sh->D, G);
    const long long cb = (target + items - 1) / items;
    if (cb > c) c = cb;
  }
  if (c > kAutoMaxChunks) c = kAutoMaxChunks;
  if (c > pages_per_split) c = pages_per_split;
  return c < 1 ? 1 : (int)c;
}

// Target kept pages per piece: a typical split (the table width over the
// split count) cut into `chunks`; a split with K kept pages is cut into
// about K / T pieces (at most `chunks`), so the splits of block-sparse heads
// are cut less than those of dense heads.
int piece_pages(const da_shape* sh, int chunks) {
  long long per_split = sh->max_pages / sh->max_splits;
  if (per_split < 1) per_split = 1;
  const long long T = (per_split + chunks - 1) / chunks;
  return T < 1 ? 1 : (int)T;
}

size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Workspace layout: the work-queue counters of the persistent launch
// (da::kQueueBytes), then, when splits are cut into chunks, chunk MA
// [n, chunks, D] and chunk m and e [n, chunks], n = S * Hq * max_splits,
// each part 16-byte aligned.
struct WsLayout {
  size_t queue, ma, m, e, total;
};

WsLayout ws_layout(const da_shape* sh, int chunks) {
  constexpr size_t Q = da::kQueueBytes;
  WsLayout w{0, Q, Q, Q, Q};
  if (chunks <= 1) return w;
  const size_t n = (size_t)sh->S * sh->Hq * sh->max_splits * chunks;
  w.ma = Q;
  w.m = w.ma + align16(n * sh->D * sizeof(float));
  w.e = w.m + align16(n * sizeof(float));
  w.total = w.e + align16(n * sizeof(float));
  return w;
}

// Workspace of the fused entry points: the group counters [S * Hkv] int32
// first (zero before the first call, left zero by every call), the work-queue
// counters, then the partials MA [n, D], m [n], e [n] with
// n = S * Hq * max_splits * chunks, each part 16-byte aligned.
WsLayout ws_fused_layout(const da_shape* sh, int chunks, size_t* counters) {
  *counters = align16((size_t)sh->S * sh->Hkv * sizeof(int32_t));
  WsLayout w{};
  w.queue = *counters;
  w.ma = w.queue + da::kQueueBytes;
  const size_t n = (size_t)sh->S * sh->Hq * sh->max_splits * chunks;
  w.m = w.ma + align16(n * sh->D * sizeof(float));
  w.e = w.m + align16(n * sizeof(float));
  w.total = w.e + align16(n * sizeof(float));
  return w;
}

// Shape checks of the page-selection entry points.
da_status check_selector(const da_shape* sh, int logical) {
  if (sh == nullptr) return fail(DA_ERR_INVALID_ARG, "shape is NULL");
  if (sh->S < 1 || sh->Hq < 1 || sh->Hkv < 1 || sh->D < 1 || sh->P < 1 || sh->max_pages < 1 ||
      sh->NP < 1)
    return fail(DA_ERR_INVALID_ARG, "sizes must be >= 1 (S=%d Hq=%d Hkv=%d D=%d P=%d max_pages=%d NP=%lld)",
                sh->S, sh->Hq, sh->Hkv, sh->D, sh->P, sh->max_pages, (long long)sh->NP);
  if (sh->Hq % sh->Hkv != 0)
    return fail(DA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", sh->Hq, sh->Hkv);
  if (sh->dtype != DA_F32 && sh->dtype != DA_BF16)
    return fail(DA_ERR_INVALID_ARG, "dtype %d is not a da_dtype", sh->dtype);
  if (sh->pool_layout != DA_POOL_PAGE_MAJOR && sh->pool_layout != DA_POOL_HEAD_MAJOR)
    return fail(DA_ERR_INVALID_ARG, "pool_layout %d is not a da_pool_layout", sh->pool_layout);
  if ((long long)sh->max_pages * sh->P > (long long)INT_MAX - sh->P)
    return fail(DA_ERR_INVALID_ARG, "max_pages * P + P exceeds the int32 token range");
  if (sh->NP > (long long)INT_MAX + 1)
    return fail(DA_ERR_INVALID_ARG, "NP exceeds the int32 block-table range");
  if (!da::selector_supported(sh->dtype, sh->D, sh->Hq / sh->Hkv, sh->P, logical))
    return fail(DA_ERR_UNSUPPORTED,
                "page selection not built for dtype=%d D=%d G=%d P=%d logical=%d", sh->dtype,
                sh->D, sh->Hq / sh->Hkv, sh->P, logical);
  if ((long long)sh->S * sh->max_pages > INT_MAX ||
      da::score_launch_items(sh->S, sh->Hkv, sh->max_pages, sh->P, logical) > INT_MAX)
    return fail(DA_ERR_INVALID_ARG, "S * max_pages exceeds the launch range");
  return DA_OK;
}

da::SelectorParams selector_params(const da_shape* sh, int logical) {
  da::SelectorParams p{};
  p.NP = sh->NP;
  p.S = sh->S;
  p.Hq = sh->Hq;
  p.Hkv = sh->Hkv;
  p.P = sh->P;
  p.max_pages = sh->max_pages;
  p.logical = logical;
  p.head_major = sh->pool_layout == DA_POOL_HEAD_MAJOR;
  return p;
}

}  // namespace

namespace {

// D, P and group size among the MicroAttention kernels built.
da_status check_micro_built(const da_shape* sh) {
  if (sh->D != 64 && sh->D != 128)
    return fail(DA_ERR_UNSUPPORTED, "head dim %d not built (64, 128)", sh->D);
  if (sh->P != 16 && sh->P != 32 && sh->P != 64 && sh->P != 128 && sh->P != 256)
    return fail(DA_ERR_UNSUPPORTED, "page size %d not built (16, 32, 64, 128, 256)", sh->P);
  const int G = sh->Hq / sh->Hkv;
  if (!da::micro_supported(sh->dtype, sh->D, G))
    return fail(DA_ERR_UNSUPPORTED, "query group size %d not built (1, 2, 4, 8)", G);
  if (sh->dtype == DA_FP4_E2M1 && sh->D == 64 && sh->P < 32 && G == 1)
    return fail(DA_ERR_UNSUPPORTED, "4-bit pages with D = 64 need P >= 32 (a wave load is 32 rows)");
  return DA_OK;
}

// Body of the MicroAttention entry points; ks / vs are the per-row scales
// of 8-bit pages (null otherwise).  out == null: partials into MA, m, e
// (chunk partials folded by the combine kernel); out != null: the fused
// step, partials in the workspace and the merge done by the last item of
// each (request, KV head), attention output into out.
da_status micro_attention_impl(const da_shape* sh, const void* q, const void* k_pages,
                               const void* v_pages, const float* ks, const float* vs,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* split_bounds, const uint8_t* block_mask, float* MA,
                               float* m, float* e, float* out, void* workspace,
                               size_t workspace_bytes, hipStream_t stream,
                               bool clear_counters = false) {
  const bool fused = out != nullptr;
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !split_bounds ||
      (!fused && (!MA || !m || !e)))
    return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) ||
      (!fused && !aligned(MA, 16)))
    return fail(DA_ERR_INVALID_ARG, "q, k_pages, v_pages and MA must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(split_bounds, 4) ||
      (!fused && (!aligned(m, 4) || !aligned(e, 4))) || (fused && !aligned(out, 4)))
    return fail(DA_ERR_INVALID_ARG, "int32/float arrays must be 4-byte aligned");
  const da_status built = check_micro_built(sh);
  if (built != DA_OK) return built;

  int chunks = resolve_chunks(sh);
  const size_t have = workspace == nullptr ? (size_t)0 : workspace_bytes;
  size_t counters = 0;
  WsLayout ws = fused ? ws_fused_layout(sh, chunks, &counters) : ws_layout(sh, chunks);
  if (chunks > 1 && have < ws.total) {
    if (sh->chunks > 1)
      return fail(DA_ERR_INVALID_ARG, "chunks=%d needs a workspace of %zu bytes (got %zu)",
                  chunks, ws.total, have);
    chunks = 1;
    ws = fused ? ws_fused_layout(sh, 1, &counters) : ws_layout(sh, 1);
  }
  if (fused && have < ws.total)
    return fail(DA_ERR_INVALID_ARG, "the fused step needs a workspace of %zu bytes (got %zu)",
                ws.total, have);
  // with room for the counter the launcher may run persistently (when the
  // grid far exceeds the resident slots); without, one workgroup per item
  const bool persistent = have >= ws.total;
  if (sh->schedule == 2 && !persistent)
    return fail(DA_ERR_INVALID_ARG, "schedule=2 needs a workspace of %zu bytes (got %zu)",
                ws.total, have);
  if ((long long)sh->S * sh->Hkv * sh->max_splits * chunks > INT_MAX)
    return fail(DA_ERR_INVALID_ARG, "S * Hkv * max_splits * chunks exceeds the launch range");
  if (persistent && !aligned(workspace, 16))
    return fail(DA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  da::MicroParams p{};
  p.q = q;
  p.k = k_pages;
  p.v = v_pages;
  p.table = block_table;
  p.lens = seq_lens;
  p.bounds = split_bounds;
  p.mask = block_mask;
  p.ks = ks;
  p.vs = vs;
  char* wsb = static_cast<char*>(workspace);
  const bool in_ws = fused || chunks > 1;  // partials in the workspace
  p.MA = in_ws ? reinterpret_cast<float*>(wsb + ws.ma) : MA;
  p.m = in_ws ? reinterpret_cast<float*>(wsb + ws.m) : m;
  p.e = in_ws ? reinterpret_cast<float*>(wsb + ws.e) : e;
  p.group_count = fused ? reinterpret_cast<int*>(wsb) : nullptr;
  p.out = out;
  p.fuse = sh->fuse;
  p.chunks = chunks;
  p.piece_pages = piece_pages(sh, chunks);
  p.n_items = sh->S * sh->Hkv * sh->max_splits * chunks;
  p.schedule = sh->schedule;
  p.queue = persistent ? reinterpret_cast<int*>(wsb + ws.queue) : nullptr;
  p.S = sh->S;
  p.Hq = sh->Hq;
  p.Hkv = sh->Hkv;
  p.P = sh->P;
  p.max_pages = sh->max_pages;
  p.max_splits = sh->max_splits;
  p.bounds_per_head = sh->bounds_per_head;
  p.scale = sh->scale;
  p.NP = sh->NP;
  p.head_major = sh->pool_layout == DA_POOL_HEAD_MAJOR;
  if (fused && clear_counters) {
    const hipError_t zerr = da::launch_zero_ints(p.group_count, (long long)sh->S * sh->Hkv, stream);
    if (zerr != hipSuccess)
      return fail(DA_ERR_HIP, "counter clear launch failed: %s", hipGetErrorString(zerr));
  }
  hipError_t err = da::launch_micro(sh->dtype, sh->D, sh->Hq / sh->Hkv, p, stream);
  if (err != hipSuccess)
    return fail(DA_ERR_HIP, "micro-attention launch failed: %s", hipGetErrorString(err));
  if (chunks > 1 && !fused) {
    err = da::launch_combine(p.MA, p.m, p.e, MA, m, e, (long long)sh->S * sh->Hq * sh->max_splits,
                             chunks, sh->D, stream);
    if (err != hipSuccess)
      return fail(DA_ERR_HIP, "chunk-combine launch failed: %s", hipGetErrorString(err));
  }
  return DA_OK;
}

}  // namespace

extern "C" {

da_status da_micro_attention(const da_shape* sh, const void* q, const void* k_pages,
                             const void* v_pages, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* split_bounds,
                             const uint8_t* block_mask, float* MA, float* m, float* e,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  const da_status st = check_shape(sh);
  if (st != DA_OK) return st;
  return micro_attention_impl(sh, q, k_pages, v_pages, nullptr, nullptr, block_table, seq_lens,
                              split_bounds, block_mask, MA, m, e, nullptr, workspace,
                              workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Shared body of the quantized-page entry points: the shape must name the
// entry point's page type; out == null gives partials, else the step.
da_status quantized_step(const char* name, int32_t want, const da_shape* sh, const void* q,
                         const uint8_t* k_codes, const float* k_scales, const uint8_t* v_codes,
                         const float* v_scales, const int32_t* block_table,
                         const int32_t* seq_lens, const int32_t* split_bounds,
                         const uint8_t* block_mask, float* MA, float* m, float* e, float* out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const da_status st = check_shape(sh, true);
  if (st != DA_OK) return st;
  if (sh->dtype != want)
    return fail(DA_ERR_INVALID_ARG, "%s needs dtype %s (got %d)", name,
                want == DA_FP8_E4M3 ? "DA_FP8_E4M3" : "DA_FP4_E2M1", sh->dtype);
  if (!k_scales || !v_scales || (MA == nullptr && !out))
    return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(k_scales, 4) || !aligned(v_scales, 4))
    return fail(DA_ERR_INVALID_ARG, "scale arrays must be 4-byte aligned");
  return micro_attention_impl(sh, q, k_codes, v_codes, k_scales, v_scales, block_table, seq_lens,
                              split_bounds, block_mask, MA, m, e, out, workspace, workspace_bytes,
                              stream);
}

}  // namespace

extern "C" {

da_status da_micro_attention_fp8(const da_shape* sh, const void* q, const uint8_t* k_codes,
                                 const float* k_scales, const uint8_t* v_codes,
                                 const float* v_scales, const int32_t* block_table,
                                 const int32_t* seq_lens, const int32_t* split_bounds,
                                 const uint8_t* block_mask, float* MA, float* m, float* e,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  return quantized_step("da_micro_attention_fp8", DA_FP8_E4M3, sh, q, k_codes, k_scales, v_codes,
                        v_scales, block_table, seq_lens, split_bounds, block_mask, MA, m, e,
                        nullptr, workspace, workspace_bytes, stream);
}

da_status da_micro_attention_fp4(const da_shape* sh, const void* q, const uint8_t* k_codes,
                                 const float* k_scales, const uint8_t* v_codes,
                                 const float* v_scales, const int32_t* block_table,
                                 const int32_t* seq_lens, const int32_t* split_bounds,
                                 const uint8_t* block_mask, float* MA, float* m, float* e,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  return quantized_step("da_micro_attention_fp4", DA_FP4_E2M1, sh, q, k_codes, k_scales, v_codes,
                        v_scales, block_table, seq_lens, split_bounds, block_mask, MA, m, e,
                        nullptr, workspace, workspace_bytes, stream);
}

da_status da_micro_attention_workspace_size(const da_shape* sh, size_t* bytes) {
  g_last_error.clear();
  if (bytes == nullptr) return fail(DA_ERR_INVALID_ARG, "bytes is NULL");
  da_status st = check_shape(sh, true);
  if (st != DA_OK) return st;
  st = check_micro_built(sh);
  if (st != DA_OK) return st;
  *bytes = ws_layout(sh, resolve_chunks(sh)).total;
  return DA_OK;
}

da_status da_attention(const da_shape* sh, const void* q, const void* k_pages, const void* v_pages,
                       const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* split_bounds, const uint8_t* block_mask, float* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  const da_status st = check_shape(sh);
  if (st != DA_OK) return st;
  if (!out) return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  return micro_attention_impl(sh, q, k_pages, v_pages, nullptr, nullptr, block_table, seq_lens,
                              split_bounds, block_mask, nullptr, nullptr, nullptr, out, workspace,
                              workspace_bytes, stream);
}

da_status da_attention_fp8(const da_shape* sh, const void* q, const uint8_t* k_codes,
                           const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                           const int32_t* block_table, const int32_t* seq_lens,
                           const int32_t* split_bounds, const uint8_t* block_mask, float* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  if (!out) return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  return quantized_step("da_attention_fp8", DA_FP8_E4M3, sh, q, k_codes, k_scales, v_codes,
                        v_scales, block_table, seq_lens, split_bounds, block_mask, nullptr,
                        nullptr, nullptr, out, workspace, workspace_bytes, stream);
}

da_status da_attention_fp4(const da_shape* sh, const void* q, const uint8_t* k_codes,
                           const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                           const int32_t* block_table, const int32_t* seq_lens,
                           const int32_t* split_bounds, const uint8_t* block_mask, float* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  if (!out) return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  return quantized_step("da_attention_fp4", DA_FP4_E2M1, sh, q, k_codes, k_scales, v_codes,
                        v_scales, block_table, seq_lens, split_bounds, block_mask, nullptr,
                        nullptr, nullptr, out, workspace, workspace_bytes, stream);
}

}  // extern "C"

// Scratch of da_attention_noalloc: the counters, work queue and partials of
// the step, in device memory the library holds from load until the process
// ends (one copy per GPU), so that the entry point allocates nothing.  In
// host code `scratch` is only a stand-in for the symbol: its device address
// on each GPU comes from hipGetSymbolAddress, taken once per device.
__device__ __align__(256) unsigned char scratch[DA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // address of `scratch` on each device, or null

da_status scratch_of_current_device(void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail(DA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DA_ERR_UNSUPPORTED, "device %d beyond the %d devices the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || p == nullptr)
      return fail(DA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(err));
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return DA_OK;
}

}  // namespace

extern "C" {

da_status da_attention_noalloc(const da_shape* sh, const void* q, const void* k_pages,
                               const void* v_pages, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* split_bounds,
                               const uint8_t* block_mask, float* out, hipStream_t stream) {
  g_last_error.clear();
  da_status st = check_shape(sh);
  if (st != DA_OK) return st;
  if (!out) return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  st = check_micro_built(sh);
  if (st != DA_OK) return st;
  // the workspace the step needs, unchunked when the library's chunking
  // would not fit (as da_attention does with a workspace too small)
  size_t counters = 0;
  const int chunks = resolve_chunks(sh);
  size_t need = ws_fused_layout(sh, chunks, &counters).total;
  if (need > DA_NOALLOC_SCRATCH_BYTES && sh->chunks == 0)
    need = ws_fused_layout(sh, 1, &counters).total;
  if (need > DA_NOALLOC_SCRATCH_BYTES)
    return fail(DA_ERR_INVALID_ARG,
                "the step needs %zu bytes of scratch; da_attention_noalloc holds %zu (use "
                "da_attention with a workspace)",
                need, (size_t)DA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != DA_OK) return st;
  // the group counters are cleared by a fill kernel before every call: an
  // earlier call of another shape may have left partials where they lie
  return micro_attention_impl(sh, q, k_pages, v_pages, nullptr, nullptr, block_table, seq_lens,
                              split_bounds, block_mask, nullptr, nullptr, nullptr, out, ws,
                              DA_NOALLOC_SCRATCH_BYTES, stream, true);
}

da_status da_attention_workspace_size(const da_shape* sh, size_t* bytes, size_t* counter_bytes) {
  g_last_error.clear();
  if (bytes == nullptr) return fail(DA_ERR_INVALID_ARG, "bytes is NULL");
  da_status st = check_shape(sh, true);
  if (st != DA_OK) return st;
  st = check_micro_built(sh);
  if (st != DA_OK) return st;
  size_t counters = 0;
  *bytes = ws_fused_layout(sh, resolve_chunks(sh), &counters).total;
  if (counter_bytes != nullptr) *counter_bytes = counters;
  return DA_OK;
}

da_status da_merge(const da_shape* sh, const float* MA, const float* m, const float* e,
                   float* out, hipStream_t stream) {
  g_last_error.clear();
  if (sh == nullptr) return fail(DA_ERR_INVALID_ARG, "shape is NULL");
  if (sh->S < 1 || sh->Hq < 1 || sh->D < 1 || sh->max_splits < 1)
    return fail(DA_ERR_INVALID_ARG, "sizes must be >= 1 (S=%d Hq=%d D=%d max_splits=%d)", sh->S,
                sh->Hq, sh->D, sh->max_splits);
  if ((long long)sh->S * sh->Hq > INT_MAX)
    return fail(DA_ERR_INVALID_ARG, "S * Hq exceeds the launch range");
  if (!MA || !m || !e || !out) return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(MA, 4) || !aligned(m, 4) || !aligned(e, 4) || !aligned(out, 4))
    return fail(DA_ERR_INVALID_ARG, "float arrays must be 4-byte aligned");
  const hipError_t err =
      da::launch_merge(MA, m, e, out, sh->S, sh->Hq, sh->D, sh->max_splits, stream);
  if (err != hipSuccess) return fail(DA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(err));
  return DA_OK;
}

da_status da_merge_partials(const da_shape* sh, const float* MA, const float* m, const float* e,
                            int32_t out_splits, int32_t out_slot, float* MA_out, float* m_out,
                            float* e_out, hipStream_t stream) {
  g_last_error.clear();
  if (sh == nullptr) return fail(DA_ERR_INVALID_ARG, "shape is NULL");
  if (sh->S < 1 || sh->Hq < 1 || sh->D < 1 || sh->max_splits < 1)
    return fail(DA_ERR_INVALID_ARG, "sizes must be >= 1 (S=%d Hq=%d D=%d max_splits=%d)", sh->S,
                sh->Hq, sh->D, sh->max_splits);
  if ((long long)sh->S * sh->Hq > INT_MAX)
    return fail(DA_ERR_INVALID_ARG, "S * Hq exceeds the launch range");
  if (out_splits < 1 || out_slot < 0 || out_slot >= out_splits)
    return fail(DA_ERR_INVALID_ARG, "out_slot %d outside [0, out_splits = %d)", out_slot,
                out_splits);
  if (!MA || !m || !e || !MA_out || !m_out || !e_out)
    return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(MA, 4) || !aligned(m, 4) || !aligned(e, 4) || !aligned(MA_out, 4) ||
      !aligned(m_out, 4) || !aligned(e_out, 4))
    return fail(DA_ERR_INVALID_ARG, "float arrays must be 4-byte aligned");
  const hipError_t err = da::launch_merge_partials(MA, m, e, MA_out, m_out, e_out, sh->S, sh->Hq,
                                                   sh->D, sh->max_splits, out_splits, out_slot,
                                                   stream);
  if (err != hipSuccess)
    return fail(DA_ERR_HIP, "partial merge launch failed: %s", hipGetErrorString(err));
  return DA_OK;
}

da_status da_check_inputs(const da_shape* sh, const int32_t* block_table,
                          const int32_t* seq_lens, int32_t* err, hipStream_t stream) {
  g_last_error.clear();
  if (sh == nullptr) return fail(DA_ERR_INVALID_ARG, "shape is NULL");
  if (sh->S < 1 || sh->P < 1 || sh->max_pages < 1 || sh->NP < 1)
    return fail(DA_ERR_INVALID_ARG, "sizes must be >= 1");
  if (!block_table || !seq_lens || !err) return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(err, 4))
    return fail(DA_ERR_INVALID_ARG, "int32 arrays must be 4-byte aligned");
  if ((long long)sh->S * sh->max_pages > (long long)UINT_MAX * 256)
    return fail(DA_ERR_INVALID_ARG, "table too large");
  const hipError_t e2 = da::launch_check_inputs(block_table, seq_lens, sh->S, sh->P, sh->max_pages,
                                                sh->NP, err, stream);
  if (e2 != hipSuccess) return fail(DA_ERR_HIP, "check launch failed: %s", hipGetErrorString(e2));
  return DA_OK;
}

da_status da_page_stats(const da_shape* sh, const void* k_pages, const int32_t* block_table,
                        const int32_t* seq_lens, int32_t logical, const uint8_t* select_heads,
                        void* stats, hipStream_t stream) {
  g_last_error.clear();
  da_status st = check_selector(sh, logical);
  if (st != DA_OK) return st;
  if (!k_pages || !block_table || !seq_lens || !stats)
    return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(k_pages, 16) || !aligned(stats, 16))
    return fail(DA_ERR_INVALID_ARG, "k_pages and stats must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4))
    return fail(DA_ERR_INVALID_ARG, "int32 arrays must be 4-byte aligned");
  da::SelectorParams p = selector_params(sh, logical);
  p.k = k_pages;
  p.stats = stats;
  p.table = block_table;
  p.lens = seq_lens;
  p.select = select_heads;
  const hipError_t err = da::launch_page_stats(p, sh->dtype, sh->D, stream);
  if (err != hipSuccess) return fail(DA_ERR_HIP, "page-stats launch failed: %s", hipGetErrorString(err));
  return DA_OK;
}

da_status da_page_scores(const da_shape* sh, const void* q, const void* stats,
                         const int32_t* block_table, const int32_t* seq_lens, int32_t logical,
                         const uint8_t* select_heads, float* scores, hipStream_t stream) {
  g_last_error.clear();
  da_status st = check_selector(sh, logical);
  if (st != DA_OK) return st;
  if (!q || !stats || !block_table || !seq_lens || !scores)
    return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(q, 16) || !aligned(stats, 16))
    return fail(DA_ERR_INVALID_ARG, "q and stats must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(scores, 4))
    return fail(DA_ERR_INVALID_ARG, "int32/float arrays must be 4-byte aligned");
  da::SelectorParams p = selector_params(sh, logical);
  p.q = q;
  p.stats = const_cast<void*>(stats);
  p.table = block_table;
  p.lens = seq_lens;
  p.select = select_heads;
  p.scores = scores;
  const hipError_t err = da::launch_page_scores(p, sh->dtype, sh->D, stream);
  if (err != hipSuccess) return fail(DA_ERR_HIP, "page-score launch failed: %s", hipGetErrorString(err));
  return DA_OK;
}

da_status da_select_pages(const da_shape* sh, const float* scores, const int32_t* seq_lens,
                          int32_t budget, int32_t keep_first, int32_t keep_last, int32_t horizon,
                          const uint8_t* select_heads, uint8_t* block_mask, hipStream_t stream) {
  g_last_error.clear();
  if (sh == nullptr) return fail(DA_ERR_INVALID_ARG, "shape is NULL");
  if (sh->S < 1 || sh->Hkv < 1 || sh->P < 1 || sh->max_pages < 1)
    return fail(DA_ERR_INVALID_ARG, "sizes must be >= 1 (S=%d Hkv=%d P=%d max_pages=%d)", sh->S,
                sh->Hkv, sh->P, sh->max_pages);
  if ((long long)sh->max_pages * sh->P > (long long)INT_MAX - sh->P)
    return fail(DA_ERR_INVALID_ARG, "max_pages * P + P exceeds the int32 token range");
  if ((long long)sh->S * sh->Hkv > INT_MAX)
    return fail(DA_ERR_INVALID_ARG, "S * Hkv exceeds the launch range");
  if (sh->max_pages > da::select_max_pages())
    return fail(DA_ERR_UNSUPPORTED, "top-K selection is built for max_pages <= %d (got %d)",
                da::select_max_pages(), sh->max_pages);
  if (budget < 0 || keep_first < 0 || keep_last < 0 || horizon < 0)
    return fail(DA_ERR_INVALID_ARG, "budget, keep_first, keep_last and horizon must be >= 0");
  if (!scores || !seq_lens || !block_mask) return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(scores, 4) || !aligned(seq_lens, 4))
    return fail(DA_ERR_INVALID_ARG, "int32/float arrays must be 4-byte aligned");
  da::SelectorParams p = selector_params(sh, 0);
  p.scores = const_cast<float*>(scores);
  p.lens = seq_lens;
  p.select = select_heads;
  p.mask = block_mask;
  p.budget = budget;
  p.keep_first = keep_first;
  p.keep_last = keep_last;
  p.horizon = horizon;
  const hipError_t err = da::launch_select_pages(p, stream);
  if (err != hipSuccess) return fail(DA_ERR_HIP, "page-select launch failed: %s", hipGetErrorString(err));
  return DA_OK;
}

da_status da_append_kv(const da_shape* sh, const void* k_new, const void* v_new,
                       const int32_t* block_table, const int32_t* seq_lens, void* k_pages,
                       void* v_pages, int32_t logical, const uint8_t* select_heads, void* stats,
                       hipStream_t stream) {
  g_last_error.clear();
  if (sh == nullptr) return fail(DA_ERR_INVALID_ARG, "shape is NULL");
  if (sh->S < 1 || sh->Hkv < 1 || sh->D < 1 || sh->P < 1 || sh->max_pages < 1 || sh->NP < 1)
    return fail(DA_ERR_INVALID_ARG, "sizes must be >= 1 (S=%d Hkv=%d D=%d P=%d max_pages=%d NP=%lld)",
                sh->S, sh->Hkv, sh->D, sh->P, sh->max_pages, (long long)sh->NP);
  if (sh->dtype != DA_F32 && sh->dtype != DA_BF16)
    return fail(DA_ERR_INVALID_ARG, "dtype %d is not a da_dtype", sh->dtype);
  if (sh->pool_layout != DA_POOL_PAGE_MAJOR && sh->pool_layout != DA_POOL_HEAD_MAJOR)
    return fail(DA_ERR_INVALID_ARG, "pool_layout %d is not a da_pool_layout", sh->pool_layout);
  if ((long long)sh->max_pages * sh->P > (long long)INT_MAX - sh->P)
    return fail(DA_ERR_INVALID_ARG, "max_pages * P + P exceeds the int32 token range");
  if ((long long)sh->S * sh->Hkv > INT_MAX)
    return fail(DA_ERR_INVALID_ARG, "S * Hkv exceeds the launch range");
  if (!da::append_supported(sh->dtype, sh->D))
    return fail(DA_ERR_UNSUPPORTED, "KV append not built for dtype=%d D=%d", sh->dtype, sh->D);
  if (stats != nullptr && !da::selector_supported(sh->dtype, sh->D, 1, sh->P, logical))
    return fail(DA_ERR_UNSUPPORTED, "statistics not built for P=%d logical=%d", sh->P, logical);
  if (!k_new || !v_new || !block_table || !seq_lens || !k_pages || !v_pages)
    return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) ||
      (stats != nullptr && !aligned(stats, 16)))
    return fail(DA_ERR_INVALID_ARG, "K/V rows, pools and statistics must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4))
    return fail(DA_ERR_INVALID_ARG, "int32 arrays must be 4-byte aligned");
  da::AppendParams p{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.table = block_table;
  p.lens = seq_lens;
  p.k = k_pages;
  p.v = v_pages;
  p.stats = stats;
  p.select = select_heads;
  p.NP = sh->NP;
  p.S = sh->S;
  p.Hkv = sh->Hkv;
  p.P = sh->P;
  p.max_pages = sh->max_pages;
  p.logical = stats != nullptr ? logical : sh->P;
  p.head_major = sh->pool_layout == DA_POOL_HEAD_MAJOR;
  const hipError_t err = da::launch_append_kv(p, sh->dtype, sh->D, stream);
  if (err != hipSuccess) return fail(DA_ERR_HIP, "KV append launch failed: %s", hipGetErrorString(err));
  return DA_OK;
}

}  // extern "C"

namespace {

// Shared body of da_append_kv_fp8 (bits 8) and da_append_kv_fp4 (bits 4).
da_status append_quantized(int bits, const da_shape* sh, const void* k_new, const void* v_new,
                           const int32_t* block_table, const int32_t* seq_lens, uint8_t* k_codes,
                           float* k_scales, uint8_t* v_codes, float* v_scales, int32_t logical,
                           const uint8_t* select_heads, void* stats, hipStream_t stream) {
  if (sh == nullptr) return fail(DA_ERR_INVALID_ARG, "shape is NULL");
  if (sh->S < 1 || sh->Hkv < 1 || sh->D < 1 || sh->P < 1 || sh->max_pages < 1 || sh->NP < 1)
    return fail(DA_ERR_INVALID_ARG, "sizes must be >= 1 (S=%d Hkv=%d D=%d P=%d max_pages=%d NP=%lld)",
                sh->S, sh->Hkv, sh->D, sh->P, sh->max_pages, (long long)sh->NP);
  if (sh->dtype != DA_F32 && sh->dtype != DA_BF16)
    return fail(DA_ERR_INVALID_ARG, "dtype of the new rows must be DA_F32 or DA_BF16 (got %d)", sh->dtype);
  if (sh->pool_layout != DA_POOL_PAGE_MAJOR && sh->pool_layout != DA_POOL_HEAD_MAJOR)
    return fail(DA_ERR_INVALID_ARG, "pool_layout %d is not a da_pool_layout", sh->pool_layout);
  if ((long long)sh->max_pages * sh->P > (long long)INT_MAX - sh->P)
    return fail(DA_ERR_INVALID_ARG, "max_pages * P + P exceeds the int32 token range");
  if ((long long)sh->S * sh->Hkv > INT_MAX)
    return fail(DA_ERR_INVALID_ARG, "S * Hkv exceeds the launch range");
  if (!da::quantize_supported(sh->dtype, sh->D))
    return fail(DA_ERR_UNSUPPORTED, "%d-bit append not built for D=%d (64, 128)", bits, sh->D);
  if (stats != nullptr && !da::selector_supported(sh->dtype, sh->D, 1, sh->P, logical))
    return fail(DA_ERR_UNSUPPORTED, "statistics not built for P=%d logical=%d", sh->P, logical);
  if (stats != nullptr && !aligned(stats, 16))
    return fail(DA_ERR_INVALID_ARG, "statistics must be 16-byte aligned");
  if (!k_new || !v_new || !block_table || !seq_lens || !k_codes || !k_scales || !v_codes || !v_scales)
    return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  const size_t ca = bits == 8 ? 8 : 4;  // a lane writes 8 codes: 8 or 4 bytes
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_codes, ca) || !aligned(v_codes, ca))
    return fail(DA_ERR_INVALID_ARG, "new rows must be 16-byte and code pools %zu-byte aligned", ca);
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(k_scales, 4) || !aligned(v_scales, 4))
    return fail(DA_ERR_INVALID_ARG, "int32/float arrays must be 4-byte aligned");
  da::AppendFp8Params p{};
  p.bits = bits;
  p.k_new = k_new;
  p.v_new = v_new;
  p.table = block_table;
  p.lens = seq_lens;
  p.k_codes = k_codes;
  p.k_scales = k_scales;
  p.v_codes = v_codes;
  p.v_scales = v_scales;
  p.stats = stats;
  p.select = select_heads;
  p.NP = sh->NP;
  p.S = sh->S;
  p.Hkv = sh->Hkv;
  p.P = sh->P;
  p.max_pages = sh->max_pages;
  p.logical = stats != nullptr ? logical : sh->P;
  p.head_major = sh->pool_layout == DA_POOL_HEAD_MAJOR;
  const hipError_t err = da::launch_append_kv_fp8(p, sh->dtype, sh->D, stream);
  if (err != hipSuccess)
    return fail(DA_ERR_HIP, "%d-bit append launch failed: %s", bits, hipGetErrorString(err));
  return DA_OK;
}

}  // namespace

extern "C" {

da_status da_append_kv_fp8(const da_shape* sh, const void* k_new, const void* v_new,
                           const int32_t* block_table, const int32_t* seq_lens, uint8_t* k_codes,
                           float* k_scales, uint8_t* v_codes, float* v_scales, int32_t logical,
                           const uint8_t* select_heads, void* stats, hipStream_t stream) {
  g_last_error.clear();
  return append_quantized(8, sh, k_new, v_new, block_table, seq_lens, k_codes, k_scales, v_codes,
                          v_scales, logical, select_heads, stats, stream);
}

da_status da_append_kv_fp4(const da_shape* sh, const void* k_new, const void* v_new,
                           const int32_t* block_table, const int32_t* seq_lens, uint8_t* k_codes,
                           float* k_scales, uint8_t* v_codes, float* v_scales, int32_t logical,
                           const uint8_t* select_heads, void* stats, hipStream_t stream) {
  g_last_error.clear();
  return append_quantized(4, sh, k_new, v_new, block_table, seq_lens, k_codes, k_scales, v_codes,
                          v_scales, logical, select_heads, stats, stream);
}

da_status da_split_bounds(const da_shape* sh, const uint8_t* block_mask, const int32_t* seq_lens,
                          int32_t horizon, int32_t* split_bounds, hipStream_t stream) {
  g_last_error.clear();
  if (sh == nullptr) return fail(DA_ERR_INVALID_ARG, "shape is NULL");
  if (sh->S < 1 || sh->Hkv < 1 || sh->P < 1 || sh->max_pages < 1 || sh->max_splits < 1)
    return fail(DA_ERR_INVALID_ARG, "sizes must be >= 1 (S=%d Hkv=%d P=%d max_pages=%d max_splits=%d)",
                sh->S, sh->Hkv, sh->P, sh->max_pages, sh->max_splits);
  if ((long long)sh->max_pages * sh->P > (long long)INT_MAX - sh->P)
    return fail(DA_ERR_INVALID_ARG, "max_pages * P + P exceeds the int32 token range");
  if ((long long)sh->S * sh->Hkv > INT_MAX)
    return fail(DA_ERR_INVALID_ARG, "S * Hkv exceeds the launch range");
  if (horizon < 0) return fail(DA_ERR_INVALID_ARG, "horizon must be >= 0");
  if (!seq_lens || !split_bounds) return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(seq_lens, 4) || !aligned(split_bounds, 4))
    return fail(DA_ERR_INVALID_ARG, "int32 arrays must be 4-byte aligned");
  da::BoundsParams p{};
  p.mask = block_mask;
  p.lens = seq_lens;
  p.bounds = split_bounds;
  p.S = sh->S;
  p.Hkv = sh->Hkv;
  p.P = sh->P;
  p.max_pages = sh->max_pages;
  p.b = sh->max_splits;
  p.horizon = horizon;
  const hipError_t err = da::launch_split_bounds(p, stream);
  if (err != hipSuccess) return fail(DA_ERR_HIP, "split-bounds launch failed: %s", hipGetErrorString(err));
  return DA_OK;
}

}  // extern "C"

namespace {

// Shared body of da_quantize_rows (bits 8) and da_quantize_rows_fp4 (bits 4).
da_status quantize_rows_impl(int bits, int32_t dtype, int64_t rows, int32_t D, const void* x,
                             uint8_t* codes, float* scales, hipStream_t stream) {
  if (rows < 0 || D < 1) return fail(DA_ERR_INVALID_ARG, "rows must be >= 0 and D >= 1");
  if (dtype != DA_F32 && dtype != DA_BF16)
    return fail(DA_ERR_INVALID_ARG, "dtype %d is not DA_F32 or DA_BF16", dtype);
  if (!da::quantize_supported(dtype, D))
    return fail(DA_ERR_UNSUPPORTED, "quantization not built for D=%d (64, 128)", D);
  if (rows == 0) return DA_OK;
  if (!x || !codes || !scales) return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  const size_t ca = bits == 8 ? 8 : 4;  // a lane writes 8 codes: 8 or 4 bytes
  if (!aligned(x, 16) || !aligned(codes, ca) || !aligned(scales, 4))
    return fail(DA_ERR_INVALID_ARG, "x must be 16-byte, codes %zu-byte and scales 4-byte aligned",
                ca);
  if (da::quantize_launch_blocks(D, rows) > UINT_MAX)
    return fail(DA_ERR_INVALID_ARG, "too many rows for one launch");
  const hipError_t err = da::launch_quantize_rows(dtype, D, bits, x, codes, scales, rows, stream);
  if (err != hipSuccess) return fail(DA_ERR_HIP, "quantize launch failed: %s", hipGetErrorString(err));
  return DA_OK;
}

}  // namespace

extern "C" {

da_status da_quantize_rows(int32_t dtype, int64_t rows, int32_t D, const void* x,
                           uint8_t* codes, float* scales, hipStream_t stream) {
  g_last_error.clear();
  return quantize_rows_impl(8, dtype, rows, D, x, codes, scales, stream);
}

da_status da_quantize_rows_fp4(int32_t dtype, int64_t rows, int32_t D, const void* x,
                               uint8_t* codes, float* scales, hipStream_t stream) {
  g_last_error.clear();
  return quantize_rows_impl(4, dtype, rows, D, x, codes, scales, stream);
}

const char* da_last_error(void) { return g_last_error.c_str(); }

da_status da_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  g_last_error.clear();
  if (!src || !sink) return fail(DA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(src, 16) || bytes % 16 != 0 || bytes == 0)
    return fail(DA_ERR_INVALID_ARG, "src must be 16-byte aligned and bytes a positive multiple of 16");
  const hipError_t err = da::launch_stream_read(src, bytes, sink, stream);
  if (err != hipSuccess) return fail(DA_ERR_HIP, "stream-read launch failed: %s", hipGetErrorString(err));
  return DA_OK;
}

size_t da_stream_read_sink_words(void) { return (size_t)da::stream_read_grid(); }

}  // extern "C"
