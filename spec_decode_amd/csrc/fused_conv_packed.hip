// Launches of the fused replay+verify with the convolution prologue over a
// packed dim-first window pool (tap stride 1, channel stride RQ + 2, slot
// stride a multiple of 8 elements, 16-byte aligned base), whose windows each
// wave moves as one contiguous block. The kernel is described in
// verify_kernel.h.
#include "verify_kernel.h"

namespace kda {

hipError_t launch_verify_conv_packed(const VerifyParams& p, int tokens, bool bf16, int batch,
                                     hipStream_t stream) {
  return launch_conv_mode<CONV_PACKED>(p, tokens, bf16, batch, stream);
}

}  // namespace kda
