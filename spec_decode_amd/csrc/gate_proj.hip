// Low-rank gate projection raw_g = BF16(F_A F_B^T) (the gate projection of the
// fused page, "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.fused",
// KdaFused.kernel): F_A [tokens][128] (rows f_a_row_stride apart, e.g. a column
// slice of a packed projection row), F_B [H*128][128], raw_g [tokens][H*128].
//
// gfx950 mapping. A dense [tokens x 128] x [128 x H*128] product with K = 128, so
// BF16 MFMA (V_MFMA_F32_16X16X32_BF16, FP32 accumulation). One workgroup of 4
// waves per (head, 256 tokens). The head's F_B tile (128 x 128, 32 KiB) is
// staged once in LDS, rows padded by 16 bytes so that the 16 rows a load
// instruction reads fall in distinct banks; each wave then streams its 4 blocks
// of 16 tokens through it: B operands (F_A rows) straight from global memory,
// the next block's prefetched while the current one runs its 32 MFMAs; A
// operands (F_B rows) from LDS. Within a 32-feature group the A rows are
// permuted so that a lane's two output tiles hold 8 consecutive features of one
// token: one 16-byte store each, and each wave writes whole 256-byte rows of
// raw_g. The output is the dominant HBM traffic (2 B per element, against
// 256 B of F_A per token and 32 KiB of F_B per head, read through L2).
#include "kda_device.h"

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int GP_TOKENS = 256;             // tokens per workgroup
constexpr int GP_BLOCKS = GP_TOKENS / 64;  // 16-token blocks per wave
constexpr int GP_ROW = K + 8;              // padded LDS row of F_B, in elements

__global__ __launch_bounds__(256) void gate_proj_kernel(const uint16_t* __restrict__ f_a,
                                                        int64_t sa,
                                                        const uint16_t* __restrict__ f_b,
                                                        uint16_t* __restrict__ out,
                                                        int64_t tokens, int heads) {
  __shared__ __attribute__((aligned(16))) uint16_t fb_s[K * GP_ROW];
  const int64_t t0 = (int64_t)blockIdx.x * GP_TOKENS;
  const int h = blockIdx.y;
  const int64_t D = (int64_t)heads * K;
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int lr = lane & 15;  // A row / B column within a tile
  const int lq = lane >> 4;  // 8-wide K group within a 32-wide K step

  // B operands of a 16-token block: column n is token tb0 + n (rows past the
  // end read the last token and are not stored).
  auto load_b = [&](int64_t tb0, bf16x8 (&b)[4]) {
    int64_t t = tb0 + lr;
    t = t < tokens ? t : tokens - 1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      b[ks] = *reinterpret_cast<const bf16x8*>(f_a + t * sa + 32 * ks + 8 * lq);
  };
  bf16x8 bcur[4], bnext[4];
  const int64_t wt0 = t0 + (int64_t)wave * 16 * GP_BLOCKS;  // this wave's first token
  load_b(wt0, bcur);

  // Stage the head's F_B tile: 2048 16-byte chunks, 8 per thread.
  const uint16_t* fbh = f_b + (int64_t)h * K * K;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int chunk = tid + 256 * i;
    const int row = chunk >> 4, col = (chunk & 15) * 8;
    *reinterpret_cast<u32x4*>(&fb_s[row * GP_ROW + col]) =
        *reinterpret_cast<const u32x4*>(fbh + row * K + col);
  }
  __syncthreads();

#pragma unroll 1
  for (int blk = 0; blk < GP_BLOCKS; ++blk) {
    const int64_t tb0 = wt0 + 16 * blk;
    if (tb0 >= tokens) break;  // uniform
    if (blk + 1 < GP_BLOCKS) load_b(tb0 + 16, bnext);
    const int64_t t = tb0 + lr;
#pragma unroll
    for (int g = 0; g < 4; ++g) {  // 32-feature groups
      floatx4 acc[2];
#pragma unroll
      for (int fb = 0; fb < 2; ++fb) {
        // tile fb row m: feature 32g + 8(m/4) + 4fb + m%4
        const int f = 32 * g + 8 * (lr >> 2) + 4 * fb + (lr & 3);
        acc[fb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&fb_s[f * GP_ROW + 32 * ks + 8 * lq]);
          acc[fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bcur[ks], acc[fb], 0, 0, 0);
        }
      }
      // Lane l, value i of tile fb: feature 32g + 8(l/16) + 4fb + i, token tb0 + l%16.
      if (t < tokens) {
        u32x4 packed;
        packed[0] = pack_bf16x2(acc[0][0], acc[0][1]);
        packed[1] = pack_bf16x2(acc[0][2], acc[0][3]);
        packed[2] = pack_bf16x2(acc[1][0], acc[1][1]);
        packed[3] = pack_bf16x2(acc[1][2], acc[1][3]);
        *reinterpret_cast<u32x4*>(out + t * D + (int64_t)h * K + 32 * g + 8 * lq) = packed;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) bcur[ks] = bnext[ks];
  }
}

hipError_t launch_gate_projection(const uint16_t* f_a, int64_t sa, const uint16_t* f_b,
                                  uint16_t* out, int64_t tokens, int heads, hipStream_t stream) {
  const dim3 grid((unsigned)((tokens + GP_TOKENS - 1) / GP_TOKENS), heads);
  hipLaunchKernelGGL(gate_proj_kernel, grid, dim3(256), 0, stream, f_a, sa, f_b, out, tokens,
                     heads);
  return hipGetLastError();
}

}  // namespace kda
