/* Host-side driver for the C ABI of libda.so, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitizers.py).
 *
 * Every call below is rejected by the library's argument checks before any
 * GPU work is enqueued, or (da_micro_attention_workspace_size,
 * da_attention_workspace_size) is pure host arithmetic, so the driver runs on a machine without a GPU.  It exercises
 * the checks' arithmetic on extreme sizes and the error-message formatting;
 * the sanitizers turn any out-of-bounds access, overflow or other undefined
 * behaviour on those paths into a failed run.  The pointers are never
 * dereferenced: a call that got past its checks would launch, which is a
 * failure here too (DA_ERR_HIP or a crash without a GPU). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "da.h"

static int failures = 0;

#define FAKE ((void*)(uintptr_t)0x10000) /* aligned, never dereferenced */

static void expect(const char* what, da_status got, da_status want) {
  const char* msg = da_last_error();
  const size_t n = msg ? strlen(msg) : 0;
  if (got != want || (want != DA_OK && n == 0)) {
    fprintf(stderr, "FAIL %s: status %d (want %d), message '%s'\n", what, (int)got, (int)want,
            msg ? msg : "(null)");
    ++failures;
  }
}

static da_shape good(void) {
  da_shape s;
  memset(&s, 0, sizeof s);
  s.S = 2;
  s.Hq = 8;
  s.Hkv = 2;
  s.D = 128;
  s.P = 64;
  s.max_pages = 4;
  s.max_splits = 2;
  s.bounds_per_head = 0;
  s.dtype = DA_BF16;
  s.scale = 0.088f;
  s.NP = 8;
  s.chunks = 0;
  s.schedule = 0;
  s.pool_layout = DA_POOL_PAGE_MAJOR;
  return s;
}

static da_status micro(const da_shape* s, void* q, void* ws, size_t ws_bytes) {
  return da_micro_attention(s, q, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, ws,
                            ws_bytes, NULL);
}

int main(void) {
  da_shape s;
  size_t bytes = 0;

  /* micro-attention: shape checks, including products that overflow int32 */
  expect("null shape", micro(NULL, FAKE, NULL, 0), DA_ERR_INVALID_ARG);
  s = good(); s.S = 0;
  expect("S = 0", micro(&s, FAKE, NULL, 0), DA_ERR_INVALID_ARG);
  s = good(); s.Hq = 6; s.Hkv = 4;
  expect("Hq % Hkv", micro(&s, FAKE, NULL, 0), DA_ERR_INVALID_ARG);
  s = good(); s.max_pages = INT32_MAX; s.P = 256;
  expect("max_pages * P overflow", micro(&s, FAKE, NULL, 0), DA_ERR_INVALID_ARG);
  s = good(); s.S = INT32_MAX; s.Hkv = INT32_MAX; s.Hq = INT32_MAX; s.max_splits = INT32_MAX;
  expect("S * Hkv * b overflow", micro(&s, FAKE, NULL, 0), DA_ERR_INVALID_ARG);
  s = good(); s.NP = INT64_MAX;
  expect("NP range", micro(&s, FAKE, NULL, 0), DA_ERR_INVALID_ARG);
  s = good(); s.NP = INT64_MIN;
  expect("NP negative", micro(&s, FAKE, NULL, 0), DA_ERR_INVALID_ARG);
  s = good(); s.scale = 0.f / 0.f;
  expect("scale NaN", micro(&s, FAKE, NULL, 0), DA_ERR_INVALID_ARG);
  s = good(); s.dtype = INT32_MIN;
  expect("dtype", micro(&s, FAKE, NULL, 0), DA_ERR_INVALID_ARG);
  s = good(); s.dtype = DA_FP8_E4M3;
  expect("fp8 dtype on the bf16 entry", micro(&s, FAKE, NULL, 0), DA_ERR_INVALID_ARG);
  s = good(); s.pool_layout = 7;
  expect("pool layout", micro(&s, FAKE, NULL, 0), DA_ERR_INVALID_ARG);
  s = good(); s.chunks = 65;
  expect("chunks", micro(&s, FAKE, NULL, 0), DA_ERR_INVALID_ARG);
  s = good(); s.chunks = 4;
  expect("forced chunks without workspace", micro(&s, FAKE, NULL, 0), DA_ERR_INVALID_ARG);
  s = good(); s.schedule = -1;
  expect("schedule", micro(&s, FAKE, NULL, 0), DA_ERR_INVALID_ARG);
  s = good();
  expect("null q", micro(&s, NULL, NULL, 0), DA_ERR_INVALID_ARG);
  expect("misaligned q", micro(&s, (char*)FAKE + 2, NULL, 0), DA_ERR_INVALID_ARG);
  expect("misaligned workspace", micro(&s, FAKE, (char*)FAKE + 4, 4096), DA_ERR_INVALID_ARG);
  s = good(); s.D = 96;
  expect("D unsupported", micro(&s, FAKE, NULL, 0), DA_ERR_UNSUPPORTED);
  s = good(); s.P = 48;
  expect("P unsupported", micro(&s, FAKE, NULL, 0), DA_ERR_UNSUPPORTED);
  s = good(); s.Hq = 6;
  expect("G unsupported", micro(&s, FAKE, NULL, 0), DA_ERR_UNSUPPORTED);

  /* workspace size: pure host arithmetic, from tiny to very large shapes */
  s = good();
  expect("workspace size", da_micro_attention_workspace_size(&s, &bytes), DA_OK);
  s = good(); s.S = 1; s.Hq = 32; s.Hkv = 8; s.max_pages = 8192; s.max_splits = 16;
  expect("workspace size, few items", da_micro_attention_workspace_size(&s, &bytes), DA_OK);
  s = good(); s.S = 4096; s.Hq = 64; s.Hkv = 64; s.max_pages = 1 << 20; s.P = 16;
  s.max_splits = 64; s.chunks = 64;
  expect("workspace size, huge", da_micro_attention_workspace_size(&s, &bytes), DA_OK);
  expect("workspace size, null out", da_micro_attention_workspace_size(&s, NULL),
         DA_ERR_INVALID_ARG);

  /* 8-bit attention */
  s = good(); s.dtype = DA_FP8_E4M3;
  expect("fp8: null scales",
         da_micro_attention_fp8(&s, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE,
                                FAKE, FAKE, NULL, 0, NULL),
         DA_ERR_INVALID_ARG);
  s = good();
  expect("fp8: bf16 dtype",
         da_micro_attention_fp8(&s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE,
                                FAKE, FAKE, NULL, 0, NULL),
         DA_ERR_INVALID_ARG);

  /* the fused step (attention in one launch) */
  s = good();
  expect("fused: null out",
         da_attention(&s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, 1 << 20, NULL),
         DA_ERR_INVALID_ARG);
  expect("fused: no workspace",
         da_attention(&s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, 0, NULL),
         DA_ERR_INVALID_ARG);
  expect("fused: workspace too small",
         da_attention(&s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 64, NULL),
         DA_ERR_INVALID_ARG);
  expect("fused: misaligned workspace",
         da_attention(&s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, (char*)FAKE + 8,
                      (size_t)1 << 30, NULL),
         DA_ERR_INVALID_ARG);
  expect("fused: misaligned out",
         da_attention(&s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, (char*)FAKE + 2, FAKE,
                      (size_t)1 << 30, NULL),
         DA_ERR_INVALID_ARG);
  s = good(); s.S = INT32_MAX; s.Hkv = INT32_MAX; s.Hq = INT32_MAX; s.max_splits = INT32_MAX;
  expect("fused: S * Hkv * b overflow",
         da_attention(&s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 1 << 20, NULL),
         DA_ERR_INVALID_ARG);
  s = good(); s.dtype = DA_FP8_E4M3;
  expect("fused fp8: null scales",
         da_attention_fp8(&s, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE,
                          1 << 20, NULL),
         DA_ERR_INVALID_ARG);
  s = good();
  expect("fused fp8: bf16 dtype",
         da_attention_fp8(&s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE,
                          1 << 20, NULL),
         DA_ERR_INVALID_ARG);
  {
    size_t counters = 0;
    s = good();
    expect("fused workspace size", da_attention_workspace_size(&s, &bytes, &counters), DA_OK);
    if (counters < (size_t)s.S * s.Hkv * 4 || bytes <= counters) {
      fprintf(stderr, "FAIL fused workspace size: bytes %zu counters %zu\n", bytes, counters);
      ++failures;
    }
    expect("fused workspace size, no counters out", da_attention_workspace_size(&s, &bytes, NULL),
           DA_OK);
    s = good(); s.S = 4096; s.Hq = 64; s.Hkv = 64; s.max_pages = 1 << 20; s.P = 16;
    s.max_splits = 64; s.chunks = 64;
    expect("fused workspace size, huge", da_attention_workspace_size(&s, &bytes, &counters),
           DA_OK);
    expect("fused workspace size, null out", da_attention_workspace_size(&s, NULL, &counters),
           DA_ERR_INVALID_ARG);
  }

  /* merge and the partial fold */
  s = good(); s.max_splits = 0;
  expect("merge b = 0", da_merge(&s, FAKE, FAKE, FAKE, FAKE, NULL), DA_ERR_INVALID_ARG);
  s = good(); s.S = INT32_MAX; s.Hq = INT32_MAX;
  expect("merge S * Hq", da_merge(&s, FAKE, FAKE, FAKE, FAKE, NULL), DA_ERR_INVALID_ARG);
  s = good();
  expect("fold slot", da_merge_partials(&s, FAKE, FAKE, FAKE, 3, 3, FAKE, FAKE, FAKE, NULL),
         DA_ERR_INVALID_ARG);
  expect("fold slot min",
         da_merge_partials(&s, FAKE, FAKE, FAKE, INT32_MAX, INT32_MIN, FAKE, FAKE, FAKE, NULL),
         DA_ERR_INVALID_ARG);

  /* input validation, selection, decode-time update, quantization */
  expect("check_inputs null", da_check_inputs(&s, NULL, FAKE, FAKE, NULL), DA_ERR_INVALID_ARG);
  expect("page_stats logical",
         da_page_stats(&s, FAKE, FAKE, FAKE, 12, NULL, FAKE, NULL), DA_ERR_UNSUPPORTED);
  expect("page_scores null q",
         da_page_scores(&s, NULL, FAKE, FAKE, FAKE, 16, NULL, FAKE, NULL), DA_ERR_INVALID_ARG);
  expect("select budget",
         da_select_pages(&s, FAKE, FAKE, -1, 0, 0, 0, NULL, FAKE, NULL), DA_ERR_INVALID_ARG);
  expect("select horizon",
         da_select_pages(&s, FAKE, FAKE, 4, 0, 0, INT32_MIN, NULL, FAKE, NULL),
         DA_ERR_INVALID_ARG);
  s = good(); s.max_pages = INT32_MAX;
  expect("select too many pages",
         da_select_pages(&s, FAKE, FAKE, 4, 1, 1, 0, NULL, FAKE, NULL), DA_ERR_INVALID_ARG);
  s = good();
  expect("append null", da_append_kv(&s, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, 16, NULL, NULL, NULL),
         DA_ERR_INVALID_ARG);
  expect("append fp8 null",
         da_append_kv_fp8(&s, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 16, NULL, NULL, NULL),
         DA_ERR_INVALID_ARG);
  expect("split bounds horizon",
         da_split_bounds(&s, FAKE, FAKE, -5, FAKE, NULL), DA_ERR_INVALID_ARG);
  expect("quantize rows", da_quantize_rows(DA_BF16, -1, 128, FAKE, FAKE, FAKE, NULL),
         DA_ERR_INVALID_ARG);
  expect("quantize rows huge", da_quantize_rows(DA_BF16, INT64_MAX, 128, FAKE, FAKE, FAKE, NULL),
         DA_ERR_INVALID_ARG);
  expect("quantize D", da_quantize_rows(DA_BF16, 4, 96, FAKE, FAKE, FAKE, NULL),
         DA_ERR_UNSUPPORTED);
  expect("stream read size", da_stream_read(FAKE, 15, FAKE, NULL), DA_ERR_INVALID_ARG);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("host ABI checks passed\n");
  return 0;
}
