// Grouped-query MicroAttention on the matrix cores over 8-bit (FP8 E4M3)
// pages.  Built with -fno-honor-nans -mno-amdgpu-ieee (see the build's
// per-file flags): the kernel's inputs are finite and unread slots are never
// loaded, so no NaN reaches its arithmetic, and without IEEE-mode NaN
// quieting the DPP steps of its score maxima fold into v_max_f32_dpp.
#include "micro_attention_mfma.h"

namespace da {

hipError_t launch_micro_mfma_fp8(int D, int G, const MicroParams& p, hipStream_t stream) {
  return D == 64 ? dispatch_g<2, 64>(G, p, stream) : dispatch_g<2, 128>(G, p, stream);
}

}  // namespace da
