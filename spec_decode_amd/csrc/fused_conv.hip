// Launches of the fused replay+verify with the convolution prologue (q, k, v
// computed from the packed pre-activations and each channel's window), over
// FP32 or BF16 pages, with or without the gated RMSNorm output stage. The
// kernel is described in verify_kernel.h.
#include "verify_kernel.h"

namespace kda {

template <bool GATED, bool SB16>
static hipError_t launch_conv_t(const VerifyParams& p, int tokens, dim3 grid,
                                hipStream_t stream) {
  switch (tokens) {
#define KDA_VERIFY_CASE(TT)                                                                  \
  case TT:                                                                                  \
    hipLaunchKernelGGL((verify_kernel<TT, true, GATED, SB16, true>), grid, dim3(256), 0,    \
                       stream, p);                                                          \
    break;
    KDA_VERIFY_CASE(1)
    KDA_VERIFY_CASE(2)
    KDA_VERIFY_CASE(3)
    KDA_VERIFY_CASE(4)
    KDA_VERIFY_CASE(5)
    KDA_VERIFY_CASE(6)
    KDA_VERIFY_CASE(7)
    KDA_VERIFY_CASE(8)
#undef KDA_VERIFY_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_verify_conv(const VerifyParams& p, int tokens, bool bf16, int batch,
                              hipStream_t stream) {
  const dim3 grid(p.heads, batch);
  if (p.gate != nullptr)
    return bf16 ? launch_conv_t<true, true>(p, tokens, grid, stream)
                : launch_conv_t<true, false>(p, tokens, grid, stream);
  return bf16 ? launch_conv_t<false, true>(p, tokens, grid, stream)
              : launch_conv_t<false, false>(p, tokens, grid, stream);
}

}  // namespace kda
