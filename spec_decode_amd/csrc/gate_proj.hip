// Low-rank gate projection raw_g = BF16(F_A F_B^T) (the gate projection of the
// fused page, "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.fused",
// KdaFused.kernel): F_A [tokens][128] (rows f_a_row_stride apart, e.g. a column
// slice of a packed projection row), F_B [H*128][128], raw_g [tokens][H*128].
//
// gfx950 mapping. A dense [tokens x 128] x [128 x H*128] product with K = 128, so
// BF16 MFMA (V_MFMA_F32_16X16X32_BF16, FP32 accumulation). One workgroup of 4
// waves per (64 tokens, head): wave w owns the head's features 32w..32w+31 as
// two 16-row A tiles (F_B rows), the 64 tokens as four 16-column B tiles (F_A
// rows), and the full K = 128 as 4 MFMA steps. Within a wave the A rows are
// permuted so that a lane's two output tiles hold 8 consecutive features of one
// token: one 16-byte store per (token block, lane). The output is the dominant
// traffic (2 B per element against 256 B of F_A per token and 32 KiB of F_B per
// head, which stay in L2 across the grid).
#include "kda_device.h"

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void gate_proj_kernel(const uint16_t* __restrict__ f_a,
                                                        int64_t sa,
                                                        const uint16_t* __restrict__ f_b,
                                                        uint16_t* __restrict__ out,
                                                        int64_t tokens, int heads) {
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int h = blockIdx.y;
  const int64_t D = (int64_t)heads * K;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int lr = lane & 15;  // A row / B column within a tile
  const int lq = lane >> 4;  // 8-wide K group within a 32-wide K step

  // A tiles: tile fb row m is feature 32w + 8(m/4) + 4fb + m%4 of the head.
  bf16x8 a[2][4];
#pragma unroll
  for (int fb = 0; fb < 2; ++fb) {
    const int64_t f = (int64_t)h * K + 32 * wave + 8 * (lr >> 2) + 4 * fb + (lr & 3);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      a[fb][ks] = *reinterpret_cast<const bf16x8*>(f_b + f * K + 32 * ks + 8 * lq);
  }
  // B tiles: column n of token block tb is token t0 + 16tb + n (rows past the
  // end read the last token and are not stored).
  bf16x8 b[4][4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    int64_t t = t0 + 16 * tb + lr;
    t = t < tokens ? t : tokens - 1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      b[tb][ks] = *reinterpret_cast<const bf16x8*>(f_a + t * sa + 32 * ks + 8 * lq);
  }
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    floatx4 acc[2];
#pragma unroll
    for (int fb = 0; fb < 2; ++fb) {
      acc[fb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc[fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fb][ks], b[tb][ks], acc[fb], 0, 0,
                                                          0);
    }
    // Lane l, value i of tile fb: feature 32w + 8(l/16) + 4fb + i, token 16tb + l%16.
    const int64_t t = t0 + 16 * tb + lr;
    if (t < tokens) {
      u32x4 packed;
      packed[0] = pack_bf16x2(acc[0][0], acc[0][1]);
      packed[1] = pack_bf16x2(acc[0][2], acc[0][3]);
      packed[2] = pack_bf16x2(acc[1][0], acc[1][1]);
      packed[3] = pack_bf16x2(acc[1][2], acc[1][3]);
      *reinterpret_cast<u32x4*>(out + t * D + (int64_t)h * K + 32 * wave + 8 * lq) = packed;
    }
  }
}

hipError_t launch_gate_projection(const uint16_t* f_a, int64_t sa, const uint16_t* f_b,
                                  uint16_t* out, int64_t tokens, int heads, hipStream_t stream) {
  const dim3 grid((unsigned)((tokens + 63) / 64), heads);
  hipLaunchKernelGGL(gate_proj_kernel, grid, dim3(256), 0, stream, f_a, sa, f_b, out, tokens,
                     heads);
  return hipGetLastError();
}

}  // namespace kda
