// Launches of the fused replay+verify with the convolution prologue over a
// window-major pool (channel stride 1; tap and slot strides multiples of 8
// elements, 16-byte aligned base) with 16-byte aligned input rows: each wave
// moves its inputs, taps and new window entries as 16-byte chunks through an
// LDS stage. The kernel is described in verify_kernel.h.
#include "verify_kernel.h"

namespace kda {

hipError_t launch_verify_conv_window_major(const VerifyParams& p, int tokens, bool bf16,
                                           int batch, hipStream_t stream) {
  return launch_conv_mode<CONV_WINDOW_MAJOR>(p, tokens, bf16, batch, stream);
}

}  // namespace kda
