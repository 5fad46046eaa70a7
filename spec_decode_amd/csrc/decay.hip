// Standalone bounded gate decay over a [tokens][heads][128] BF16 raw-gate tensor
// (the vLLM page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.fused",
// KdaFused.decay). Each thread converts 8 channels: one 16-byte load, two
// 16-byte stores, fully coalesced.
#include "kda_device.h"

namespace kda {

__global__ __launch_bounds__(256) void decay_kernel(const uint16_t* __restrict__ raw_g,
                                                    int64_t chunks, int heads,
                                                    const float* __restrict__ a_log,
                                                    const float* __restrict__ dt_bias, float lb,
                                                    float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= chunks) return;
  constexpr int CPR = K / 8;  // 16-byte chunks per (token, head) row
  const int c0 = (int)(i % CPR) * 8;
  const int h = (int)((i / CPR) % heads);
  const uint4 g = reinterpret_cast<const uint4*>(raw_g)[i];
  const float ea = __expf(a_log[h]);
  const float4 b0 = reinterpret_cast<const float4*>(dt_bias + (int64_t)h * K + c0)[0];
  const float4 b1 = reinterpret_cast<const float4*>(dt_bias + (int64_t)h * K + c0)[1];
  float4 o0, o1;
  o0.x = gate_decay(bf16_lo(g.x), ea, b0.x, lb);
  o0.y = gate_decay(bf16_hi(g.x), ea, b0.y, lb);
  o0.z = gate_decay(bf16_lo(g.y), ea, b0.z, lb);
  o0.w = gate_decay(bf16_hi(g.y), ea, b0.w, lb);
  o1.x = gate_decay(bf16_lo(g.z), ea, b1.x, lb);
  o1.y = gate_decay(bf16_hi(g.z), ea, b1.y, lb);
  o1.z = gate_decay(bf16_lo(g.w), ea, b1.z, lb);
  o1.w = gate_decay(bf16_hi(g.w), ea, b1.w, lb);
  float4* dst = reinterpret_cast<float4*>(out) + 2 * i;
  dst[0] = o0;
  dst[1] = o1;
}

hipError_t launch_decay(const uint16_t* raw_g, int64_t tokens, int heads, const float* a_log,
                        const float* dt_bias, float lb, float* out, hipStream_t stream) {
  const int64_t chunks = tokens * heads * (K / 8);
  const int64_t blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL(decay_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, raw_g, chunks,
                     heads, a_log, dt_bias, lb, out);
  return hipGetLastError();
}

}  // namespace kda
