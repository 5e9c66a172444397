// Grouped-query MicroAttention on the matrix cores: launches for bf16 pages
// and the dispatch between page types (the kernel is in micro_attention_mfma.h).
#include "micro_attention_mfma.h"

namespace da {

bool micro_mfma_supported(int dtype, int D, int G) {
  return (dtype == 1 || dtype == 2 || dtype == 3) && (D == 64 || D == 128) &&
         (G == 2 || G == 4 || G == 8);
}

hipError_t launch_micro_mfma(int dtype, int D, int G, const MicroParams& p, hipStream_t stream) {
  if (dtype == 2) return launch_micro_mfma_fp8(D, G, p, stream);
  if (dtype == 3) return launch_micro_mfma_fp4(D, G, p, stream);
  return D == 64 ? dispatch_g<1, 64>(G, p, stream) : dispatch_g<1, 128>(G, p, stream);
}

}  // namespace da
