// Launches of the fused replay+verify with the convolution prologue (q, k, v
// computed from the packed pre-activations and each channel's window), over
// FP32 or BF16 pages, with or without the gated RMSNorm output stage: window
// pools of any strides here, packed dim-first pools in fused_conv_packed.hip,
// window-major pools with 16-byte aligned rows (and input rows) in
// fused_conv_window_major.hip. The kernel is described in verify_kernel.h.
#include "verify_kernel.h"

namespace kda {

hipError_t launch_verify_conv(const VerifyParams& p, int tokens, bool bf16, int batch,
                              hipStream_t stream) {
  const bool pool16 = (reinterpret_cast<uintptr_t>(p.conv) & 15) == 0 && p.conv_ss % 8 == 0;
  const bool packed = pool16 && p.conv_ts == 1 && p.conv_cs == p.rq + 2;
  if (packed) return launch_verify_conv_packed(p, tokens, bf16, batch, stream);
  // Window-major: each window entry a row of consecutive channels, every row
  // (and every input row) starting on 16 bytes.
  const bool window_major = pool16 && p.conv_cs == 1 && p.conv_ts % 8 == 0 &&
                            (reinterpret_cast<uintptr_t>(p.x) & 15) == 0 && p.x_stride % 8 == 0;
  if (window_major) return launch_verify_conv_window_major(p, tokens, bf16, batch, stream);
  return launch_conv_mode<CONV_STRIDED>(p, tokens, bf16, batch, stream);
}

}  // namespace kda
