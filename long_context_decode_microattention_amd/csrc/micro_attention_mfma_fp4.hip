// Grouped-query MicroAttention on the matrix cores over 4-bit (FP4 E2M1)
// pages.  Built with -fno-honor-nans -mno-amdgpu-ieee like the 8-bit
// instances (see the build's per-file flags): the kernel's inputs are finite
// and unread slots are never loaded, so no NaN reaches its arithmetic.
#include "micro_attention_mfma.h"

namespace da {

hipError_t launch_micro_mfma_fp4(int D, int G, const MicroParams& p, hipStream_t stream) {
  return D == 64 ? dispatch_g<3, 64>(G, p, stream) : dispatch_g<3, 128>(G, p, stream);
}

}  // namespace da
