// Launches of the verify kernel without the convolution prologue: the stock
// verify and the fused replay+verify, over FP32 or BF16 pages, with or without
// the gated RMSNorm output stage. The kernel is described in verify_kernel.h.
// The stock verify writes o and the records through the L2 (STREAM) when the
// pages it reads exceed the MALL: 1.9% (FP32) and 3.8% (BF16) faster on the
// large decode batch, at its natural occupancy.
#include "verify_kernel.h"

namespace kda {

template <bool FUSED, bool GATED, bool SB16>
static hipError_t launch_t(const VerifyParams& p, int tokens, dim3 grid, hipStream_t stream) {
  switch (tokens) {
#define KDA_VERIFY_CASE(TT)                                                                   \
  case TT:                                                                                   \
    if constexpr (FUSED)                                                                     \
      return launch_fused_instance<TT, GATED, SB16, CONV_NONE>(p, grid, stream);             \
    if (stream_pages((int64_t)grid.x * grid.y * PAGE * (SB16 ? 2 : 4)))                      \
      hipLaunchKernelGGL((verify_kernel<TT, false, GATED, SB16, CONV_NONE, true>), grid,     \
                         dim3(256), 0, stream, p);                                           \
    else                                                                                     \
      hipLaunchKernelGGL((verify_kernel<TT, false, GATED, SB16, CONV_NONE, false>), grid,    \
                         dim3(256), 0, stream, p);                                           \
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

template <bool FUSED, bool GATED>
static hipError_t launch_page(const VerifyParams& p, int tokens, bool bf16, dim3 grid,
                              hipStream_t stream) {
  return bf16 ? launch_t<FUSED, GATED, true>(p, tokens, grid, stream)
              : launch_t<FUSED, GATED, false>(p, tokens, grid, stream);
}

hipError_t launch_verify(const VerifyParams& p, int tokens, bool fused, bool bf16, int batch,
                         hipStream_t stream) {
  if (p.x != nullptr) return fused ? launch_verify_conv(p, tokens, bf16, batch, stream)
                                   : hipErrorInvalidValue;
  const dim3 grid(p.heads, batch);
  const bool gated = p.gate != nullptr;
  if (fused)
    return gated ? launch_page<true, true>(p, tokens, bf16, grid, stream)
                 : launch_page<true, false>(p, tokens, bf16, grid, stream);
  return gated ? launch_page<false, true>(p, tokens, bf16, grid, stream)
               : launch_page<false, false>(p, tokens, bf16, grid, stream);
}

}  // namespace kda
