// Standalone bounded gate decay over a [tokens][heads][128] BF16 raw-gate tensor
// (the vLLM page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.fused",
// KdaFused.decay). Each thread converts 4 channels at a time: one 8-byte load
// and one 16-byte store, so every store instruction of a wave writes 1 KiB of
// contiguous output (with 8 channels per thread, two 16-byte stores at a
// 32-byte stride each covered every other 16 bytes, 5% slower). The grid is
// capped at 64 workgroups per CU and each thread strides over the chunks: on
// the large decode batch's 4096 x 64 x 128 gates (two chunks per thread) that
// takes 37.1-37.4 us against 40.4-40.8 us with one workgroup per 256 chunks.
#include <algorithm>

#include "kda_device.h"

namespace kda {

constexpr int64_t DECAY_MAX_BLOCKS = 256 * 64;

__global__ __launch_bounds__(256) void decay_kernel(const uint16_t* __restrict__ raw_g,
                                                    int64_t chunks, int heads,
                                                    const float* __restrict__ a_log,
                                                    const float* __restrict__ dt_bias, float lb,
                                                    float* __restrict__ out) {
  constexpr int CPR = K / 4;  // 8-byte chunks per (token, head) row
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < chunks; i += step) {
    const int c0 = (int)(i % CPR) * 4;
    const int h = (int)((i / CPR) % heads);
    const uint2 g = reinterpret_cast<const uint2*>(raw_g)[i];
    const float ea = __expf(a_log[h]);
    const float4 b = *reinterpret_cast<const float4*>(dt_bias + (int64_t)h * K + c0);
    float4 o;
    o.x = gate_decay(bf16_lo(g.x), ea, b.x, lb);
    o.y = gate_decay(bf16_hi(g.x), ea, b.y, lb);
    o.z = gate_decay(bf16_lo(g.y), ea, b.z, lb);
    o.w = gate_decay(bf16_hi(g.y), ea, b.w, lb);
    reinterpret_cast<float4*>(out)[i] = o;
  }
}

hipError_t launch_decay(const uint16_t* raw_g, int64_t tokens, int heads, const float* a_log,
                        const float* dt_bias, float lb, float* out, hipStream_t stream) {
  const int64_t chunks = tokens * heads * (K / 4);
  const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, DECAY_MAX_BLOCKS);
  hipLaunchKernelGGL(decay_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, raw_g, chunks,
                     heads, a_log, dt_bias, lb, out);
  return hipGetLastError();
}

}  // namespace kda
