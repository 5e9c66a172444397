// Internal kernel-launch interface of libda.so (host side of the kernels).
// The public C ABI in include/da.h validates arguments and then calls these.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace da {

struct MicroParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* table;
  const int32_t* lens;
  const int32_t* bounds;
  const uint8_t* mask;  // may be null
  const float* ks;      // fp8 pages: per-(page, head, slot) scales of K and V, else null
  const float* vs;
  float* MA;  // [S, Hq, max_splits, chunks, D]: the split partials when chunks == 1,
  float* m;   // else one partial per chunk (workspace), folded by launch_combine
  float* e;
  int S, Hq, Hkv, P, max_pages, max_splits, bounds_per_head;
  int chunks;       // pieces per split, >= 1 (plan_piece)
  int piece_pages;  // T: target kept pages per piece, >= 1
  float scale;
  long long NP;     // pages in the pools
  int head_major;   // 0: pools [NP, Hkv, P, D] (scales [NP, Hkv, P]); 1: [Hkv, NP, P, D] ([Hkv, NP, P])
  // Persistent launch: `queue` holds kQueues counters, kQueueStride ints
  // apart, all zero when the kernel starts (kQueueBytes of workspace);
  // counter q hands out, one at a time, the items of the splits j with
  // j % kQueues == q, and a workgroup takes from the queue of its own XCD
  // first (for_each_item) until all n_items = S*Hkv*max_splits*chunks are
  // taken.  queue == null: one workgroup per item (grid = n_items).
  int* queue;
  int n_items;
  int schedule;  // 0: launcher's choice, 1: one workgroup per item, 2: persistent
  // Fused merge: group_count [S * Hkv] counters, zero when the kernel starts
  // and left zero by it; the item completing the last partial of its
  // (request, KV head) merges the group's partials into out [S, Hq, D].
  // group_count == null: partials only.
  int* group_count;
  float* out;
  int fuse;  // with group_count: 0 launcher's choice, 1 one launch, 2 plain kernel + merge kernel
};

// Returns hipErrorInvalidValue for a (dtype, D, G) combination that is not
// built; callers check the combination before calling.
hipError_t launch_micro(int dtype, int D, int G, const MicroParams& p, hipStream_t stream);
bool micro_supported(int dtype, int D, int G);
// Workgroups a launch of that kernel wants for balance (the chunk heuristic's
// target): the matrix-core kernel holds fewer workgroups per CU and gains
// from finer pieces.
long long micro_target_items(int dtype, int D, int G);
bool micro_mfma_supported(int dtype, int D, int G);  // the GQA matrix-core kernel runs it

// Folds `chunks` partials per (request, head, split) into one:
// cMA [n, chunks, D], cm/ce [n, chunks] -> MA [n, D], m/e [n], n = S*Hq*max_splits.
// Zeroes the persistent-launch counter (a one-lane kernel, not a memset, so
// it can be captured in a graph).
// The persistent launch's work queues: one counter per XCD, each in its own
// 64-byte line.
constexpr int kQueues = 8;
constexpr int kQueueStride = 16;  // ints
constexpr size_t kQueueBytes = (size_t)kQueues * kQueueStride * sizeof(int);
hipError_t launch_queue_reset(int* queue, hipStream_t stream);
// Zeroes n ints with a fill kernel (capturable in a graph, unlike a memset node).
hipError_t launch_zero_ints(int* p, long long n, hipStream_t stream);

hipError_t launch_combine(const float* cMA, const float* cm, const float* ce, float* MA, float* m,
                          float* e, long long n, int chunks, int D, hipStream_t stream);

hipError_t launch_merge(const float* MA, const float* m, const float* e, float* out, int S, int Hq,
                        int D, int B, hipStream_t stream);

hipError_t launch_merge_partials(const float* MA, const float* m, const float* e, float* MA_out,
                                 float* m_out, float* e_out, int S, int Hq, int D, int B,
                                 int out_splits, int slot, hipStream_t stream);

hipError_t launch_check_inputs(const int32_t* table, const int32_t* lens, int S, int P,
                               int max_pages, int64_t NP, int32_t* err, hipStream_t stream);

// Page selection (selector.hip).
struct SelectorParams {
  const void* q;      // [S, Hq, D]
  const void* k;      // [NP, Hkv, P, D]
  void* stats;        // [Hkv, NP, P / logical, 2, D]
  const int32_t* table;
  const int32_t* lens;
  const uint8_t* select;  // [Hkv] or null
  float* scores;      // [S, Hkv, max_pages]
  uint8_t* mask;      // [S, Hkv, max_pages]
  long long NP;
  int S, Hq, Hkv, P, max_pages, logical;
  int budget, keep_first, keep_last, horizon;
  int head_major;     // K pool [Hkv, NP, P, D] instead of [NP, Hkv, P, D]
};
bool selector_supported(int dtype, int D, int G, int P, int logical);
hipError_t launch_page_stats(const SelectorParams& p, int dtype, int D, hipStream_t stream);
hipError_t launch_page_scores(const SelectorParams& p, int dtype, int D, hipStream_t stream);
hipError_t launch_select_pages(const SelectorParams& p, hipStream_t stream);
long long score_launch_items(int S, int Hkv, int max_pages, int P, int logical);
int select_max_pages();

// Decode-time cache update and split planning (decode_update.hip).
struct AppendParams {
  const void* k_new;  // [S, Hkv, D]
  const void* v_new;  // [S, Hkv, D]
  const int32_t* table;
  const int32_t* lens;
  void* k;            // [NP, Hkv, P, D]
  void* v;
  void* stats;        // [Hkv, NP, P / logical, 2, D] or null
  const uint8_t* select;
  long long NP;
  int S, Hkv, P, max_pages, logical;
  int head_major;     // pools [Hkv, NP, P, D] instead of [NP, Hkv, P, D]
};
struct AppendFp8Params {
  int bits;           // 8: FP8 E4M3 code rows of D bytes; 4: FP4 E2M1 rows of D / 2 bytes
  const void* k_new;  // [S, Hkv, D], bf16 or fp32
  const void* v_new;
  const int32_t* table;
  const int32_t* lens;
  uint8_t* k_codes;   // [NP, Hkv, P, D]
  float* k_scales;    // [NP, Hkv, P]
  uint8_t* v_codes;
  float* v_scales;
  void* stats;        // [Hkv, NP, P / logical, 2, D] of the new rows' dtype, or null
  const uint8_t* select;
  long long NP;
  int S, Hkv, P, max_pages, logical;
  int head_major;     // pools and scales [Hkv, NP, P(, D)] instead of [NP, Hkv, P(, D)]
};
struct BoundsParams {
  const uint8_t* mask;  // [S, Hkv, max_pages] or null (every page kept)
  const int32_t* lens;
  int32_t* bounds;      // [S, Hkv, b + 1]
  int S, Hkv, P, max_pages, b, horizon;
};
bool append_supported(int dtype, int D);
hipError_t launch_append_kv(const AppendParams& p, int dtype, int D, hipStream_t stream);
hipError_t launch_append_kv_fp8(const AppendFp8Params& p, int dtype, int D, hipStream_t stream);
hipError_t launch_split_bounds(const BoundsParams& p, hipStream_t stream);

// 8-bit KV rows (quant.hip).
bool quantize_supported(int dtype, int D);
// bits 8: codes [rows, D] OCP FP8 E4M3; bits 4: [rows, D / 2] OCP FP4 E2M1, two per byte.
hipError_t launch_quantize_rows(int dtype, int D, int bits, const void* x, uint8_t* codes,
                                float* scales, long long rows, hipStream_t stream);
long long quantize_launch_blocks(int D, long long rows);

int stream_read_grid();
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace da
