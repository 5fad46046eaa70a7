// Low-rank gate projection raw_g = BF16(F_A F_B^T) (the gate projection of the
// fused page, "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.fused",
// KdaFused.kernel): F_A [tokens][128] (rows f_a_row_stride apart, e.g. a column
// slice of a packed projection row), F_B [H*128][128], raw_g [tokens][H*128].
//
// gfx950 mapping. A dense [tokens x 128] x [128 x H*128] product with K = 128, so
// BF16 MFMA (V_MFMA_F32_16X16X32_BF16, FP32 accumulation). One workgroup of 4
// waves per (128 tokens, group of 4 heads). Each wave loads the B operands of
// its 32 tokens (F_A rows, two 16-token blocks) once and keeps them in
// registers for all the group's heads, so F_A crosses L2 once per head group
// instead of once per head. The heads' F_B tiles (128 x 128, 32 KiB each, rows
// padded by 16 bytes so that the 16 rows a load instruction reads fall in
// distinct banks) stream through two LDS buffers: the next head's tile is
// loaded into registers while the current one is used, then stored to the
// other buffer. Each A fragment (F_B rows) read from LDS serves both token
// blocks. Within a 32-feature group the A rows are permuted so that a lane's
// two output tiles hold 8 consecutive features of one token: one 16-byte store
// each. The output is the dominant HBM traffic (2 B per element, against
// 256 B of F_A per token and head group and 32 KiB of F_B per head and token
// group, read through L2).
#include "kda_device.h"

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int GP_TOKENS = 128;            // tokens per workgroup
constexpr int GP_HEADS = 4;               // heads per workgroup
constexpr int GP_BLOCKS = GP_TOKENS / 64; // 16-token blocks per wave
constexpr int GP_ROW = K + 8;             // padded LDS row of F_B, in elements

__global__ __launch_bounds__(256) void gate_proj_kernel(const uint16_t* __restrict__ f_a,
                                                        int64_t sa,
                                                        const uint16_t* __restrict__ f_b,
                                                        uint16_t* __restrict__ out,
                                                        int64_t tokens, int heads) {
  __shared__ __attribute__((aligned(16))) uint16_t fb_s[2][K * GP_ROW];
  const int64_t t0 = (int64_t)blockIdx.x * GP_TOKENS;
  const int h0 = blockIdx.y * GP_HEADS;
  const int nh = heads - h0 < GP_HEADS ? heads - h0 : GP_HEADS;  // heads of this group
  const int64_t D = (int64_t)heads * K;
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int lr = lane & 15;  // A row / B column within a tile
  const int lq = lane >> 4;  // 8-wide K group within a 32-wide K step
  const int64_t wt0 = t0 + (int64_t)wave * 16 * GP_BLOCKS;  // this wave's first token

  // B operands of the wave's blocks: column n of block blk is token
  // wt0 + 16 blk + n (rows past the end read the last token and are not stored).
  bf16x8 bb[GP_BLOCKS][4];
#pragma unroll
  for (int blk = 0; blk < GP_BLOCKS; ++blk) {
    int64_t t = wt0 + 16 * blk + lr;
    t = t < tokens ? t : tokens - 1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      bb[blk][ks] = *reinterpret_cast<const bf16x8*>(f_a + t * sa + 32 * ks + 8 * lq);
  }

  // A head's F_B tile: 2048 16-byte chunks, 8 per thread, through registers.
  u32x4 stage[8];
  auto load_tile = [&](int h) {
    const uint16_t* fbh = f_b + (int64_t)h * K * K;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int chunk = tid + 256 * i;
      stage[i] = *reinterpret_cast<const u32x4*>(fbh + (chunk >> 4) * K + (chunk & 15) * 8);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int chunk = tid + 256 * i;
      *reinterpret_cast<u32x4*>(&fb_s[buf][(chunk >> 4) * GP_ROW + (chunk & 15) * 8]) =
          stage[i];
    }
  };
  load_tile(h0);
  store_tile(0);
  __syncthreads();

#pragma unroll 1
  for (int hh = 0; hh < nh; ++hh) {
    const int h = h0 + hh;
    const int buf = hh & 1;
    if (hh + 1 < nh) load_tile(h + 1);  // lands while this head is computed
#pragma unroll
    for (int g = 0; g < 4; ++g) {  // 32-feature groups
      floatx4 acc[GP_BLOCKS][2];
#pragma unroll
      for (int blk = 0; blk < GP_BLOCKS; ++blk)
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) acc[blk][fb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int fb = 0; fb < 2; ++fb) {
        // tile fb row m: feature 32g + 8(m/4) + 4fb + m%4
        const int f = 32 * g + 8 * (lr >> 2) + 4 * fb + (lr & 3);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(&fb_s[buf][f * GP_ROW + 32 * ks + 8 * lq]);
#pragma unroll
          for (int blk = 0; blk < GP_BLOCKS; ++blk)
            acc[blk][fb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb[blk][ks], acc[blk][fb], 0, 0, 0);
        }
      }
      // Lane l, value i of tile fb: feature 32g + 8(l/16) + 4fb + i, token of column l%16.
#pragma unroll
      for (int blk = 0; blk < GP_BLOCKS; ++blk) {
        const int64_t t = wt0 + 16 * blk + lr;
        if (t < tokens) {
          u32x4 packed;
          packed[0] = pack_bf16x2(acc[blk][0][0], acc[blk][0][1]);
          packed[1] = pack_bf16x2(acc[blk][0][2], acc[blk][0][3]);
          packed[2] = pack_bf16x2(acc[blk][1][0], acc[blk][1][1]);
          packed[3] = pack_bf16x2(acc[blk][1][2], acc[blk][1][3]);
          *reinterpret_cast<u32x4*>(out + t * D + (int64_t)h * K + 32 * g + 8 * lq) = packed;
        }
      }
    }
    if (hh + 1 < nh) {
      // The other buffer was last read for head hh - 1, before the barrier
      // that ended that head.
      store_tile(buf ^ 1);
      __syncthreads();
    }
  }
}

hipError_t launch_gate_projection(const uint16_t* f_a, int64_t sa, const uint16_t* f_b,
                                  uint16_t* out, int64_t tokens, int heads, hipStream_t stream) {
  const dim3 grid((unsigned)((tokens + GP_TOKENS - 1) / GP_TOKENS),
                  (unsigned)((heads + GP_HEADS - 1) / GP_HEADS));
  hipLaunchKernelGGL(gate_proj_kernel, grid, dim3(256), 0, stream, f_a, sa, f_b, out, tokens,
                     heads);
  return hipGetLastError();
}

}  // namespace kda
