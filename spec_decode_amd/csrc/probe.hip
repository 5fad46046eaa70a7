// Measurement aid: the in-place read+write ceiling of the state pool in the
// access pattern the fused kernel uses on pools larger than the MALL. Every
// page of every named slot is loaded as contiguous 1 KiB pieces per wave
// instruction (no-reuse hint), turned into the 16x16 tile layout through a
// per-wave LDS area, and stored back unchanged in tile order with
// write-through, no-reuse stores (sc1 nt), one 256-thread workgroup per
// (head, request) at two workgroups per CU. The bytes moved per page equal
// the fused kernel's page traffic, with none of its arithmetic.
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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  float* page = state + (int64_t)slot * slot_stride + (int64_t)h * PAGE;
  __shared__ __attribute__((aligned(16))) u32x4 xt_s[4][16 * 32];
  u32x4 cont[16];
  load_page_contig(page, wave, lane, cont);
  u32x4 st[2][8];
  transpose_page(cont, &xt_s[wave][0], lane, st);
  // The values are opaque to the compiler (otherwise storing back what was just
  // loaded from the same address is a dead store and nothing would run).
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) asm volatile("" : "+v"(st[r][cb]));
  const __amdgpu_buffer_rsrc_t page_rs = page_rsrc(page, PAGE * 4);
  const uint32_t tile_off = (uint32_t)(((16 * (2 * wave) + (lane & 15)) * K + 4 * (lane >> 4)) * 4);
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      store_page16<CPOL_NT | CPOL_SC1>(st[r][cb], page_rs, tile_off + (16 * r * K + 16 * cb) * 4);
}

hipError_t launch_page_rw(float* state, int64_t slot_stride, const int32_t* slots, int batch,
                          int heads, int null_slot, hipStream_t stream) {
  // Dynamic LDS that leaves room for two workgroups per CU, not three.
  static const size_t pad = two_per_cu_lds(&page_rw_kernel);
  hipLaunchKernelGGL(page_rw_kernel, dim3(heads, batch), dim3(256), pad, stream, state,
                     slot_stride, slots, null_slot);
  return hipGetLastError();
}

}  // namespace kda
