// Measurement aid: the in-place read+write ceiling of the state pool in the
// access pattern the fused kernel uses. Every page of every named slot is
// loaded as 16x16 tiles (one 16-byte load per lane and tile) and stored back
// unchanged, one 256-thread workgroup per (head, request), so the bytes moved
// per page equal the fused kernel's page traffic with none of its arithmetic.
// As in the fused kernel on pools larger than the MALL, the pages go back
// through write-through, no-reuse stores (sc1 nt) at two workgroups per CU.
#include "kda_device.h"

namespace kda {

__global__ __launch_bounds__(256) void page_rw_kernel(float* __restrict__ state,
                                                      int64_t slot_stride,
                                                      const int32_t* __restrict__ slots,
                                                      int null_slot) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int slot = slots[b];
  if (slot <= null_slot) return;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  float* page = state + (int64_t)slot * slot_stride + (int64_t)h * PAGE;
  float* tile0 = page + (16 * (2 * wave) + (lane & 15)) * K + 4 * (lane >> 4);
  floatx4 st[2][8];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      st[r][cb] = *reinterpret_cast<const floatx4*>(tile0 + 16 * r * K + 16 * cb);
  // The values are opaque to the compiler (otherwise storing back what was just
  // loaded from the same address is a dead store and nothing would run).
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) asm volatile("" : "+v"(st[r][cb]));
  const __amdgpu_buffer_rsrc_t page_rs = page_rsrc(page, PAGE * 4);
  const uint32_t tile_off = (uint32_t)((tile0 - page) * 4);
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      store_page16<CPOL_NT | CPOL_SC1>(__builtin_bit_cast(u32x4, st[r][cb]), page_rs,
                                       tile_off + (16 * r * K + 16 * cb) * 4);
}

hipError_t launch_page_rw(float* state, int64_t slot_stride, const int32_t* slots, int batch,
                          int heads, int null_slot, hipStream_t stream) {
  // Dynamic LDS that leaves room for two workgroups per CU (160 KiB), not three.
  constexpr size_t TWO_PER_CU = 160 * 1024 / 3 + 256;
  hipLaunchKernelGGL(page_rw_kernel, dim3(heads, batch), dim3(256), TWO_PER_CU, stream, state,
                     slot_stride, slots, null_slot);
  return hipGetLastError();
}

}  // namespace kda
