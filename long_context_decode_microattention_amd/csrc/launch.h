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
  float* MA;
  float* m;
  float* e;
  int S, Hq, Hkv, P, max_pages, max_splits, bounds_per_head;
  float scale;
};

// Returns hipErrorInvalidValue for a (dtype, D, G) combination that is not
// built; callers check the combination before calling.
hipError_t launch_micro(int dtype, int D, int G, const MicroParams& p, hipStream_t stream);
bool micro_supported(int dtype, int D, int G);

hipError_t launch_merge(const float* MA, const float* m, const float* e, float* out, int S, int Hq,
                        int D, int B, hipStream_t stream);

hipError_t launch_check_inputs(const int32_t* table, const int32_t* lens, int S, int P,
                               int max_pages, int64_t NP, int32_t* err, hipStream_t stream);

int stream_read_grid();
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace da
