// Plan steps of deferred RecoverSSM: one thread per request.
//
// Defer: the vLLM page "vllm.models.kimi_k3.nvidia.specialized_decode.
// recoverssm.kernels", _defer_commit_kernel. Flush plan: the same page,
// _prepare_flush_plan_kernel.
#include "kda_device.h"

namespace kda {

__global__ __launch_bounds__(256) void defer_kernel(int batch, const int32_t* __restrict__ si,
                                                    int32_t* __restrict__ lens,
                                                    const int32_t* __restrict__ rows,
                                                    int32_t* __restrict__ pending,
                                                    const int32_t* __restrict__ eager,
                                                    int null_slot) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int rec = rows[b];
  if (rec < 0 || si[b] <= null_slot) return;  // padding or no record row: untouched
  if (eager != nullptr && eager[b] != 0) {
    pending[rec] = 0;  // committed now by the caller: nothing pending
  } else {
    pending[rec] = lens[b];
    lens[b] = 0;  // no commit runs for this request
  }
}

__global__ __launch_bounds__(256) void flush_plan_kernel(
    int batch, int spec_query_len, const int32_t* __restrict__ si,
    const int32_t* __restrict__ rows, const int32_t* __restrict__ pending,
    int32_t* __restrict__ lens, int32_t* __restrict__ final_idx, int32_t* __restrict__ bnd,
    int32_t* __restrict__ blens, int null_slot) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int src = si[b];
  const int rec = rows[b];
  int n = rec >= 0 ? pending[rec] : 0;
  n = min(max(n, 0), spec_query_len);
  lens[b] = (src > null_slot && n > 0) ? n : 0;
  final_idx[b] = src;
  bnd[b] = null_slot;
  blens[b] = 0;
}

hipError_t launch_defer(int batch, const int32_t* state_indices, int32_t* commit_lens,
                        const int32_t* record_rows, int32_t* pending, const int32_t* eager,
                        int null_slot, hipStream_t stream) {
  const int blocks = (batch + 255) / 256;
  hipLaunchKernelGGL(defer_kernel, dim3(blocks), dim3(256), 0, stream, batch, state_indices,
                     commit_lens, record_rows, pending, eager, null_slot);
  return hipGetLastError();
}

hipError_t launch_flush_plan(int batch, int spec_query_len, const int32_t* state_indices,
                             const int32_t* record_rows, const int32_t* pending,
                             int32_t* commit_lens, int32_t* final_indices, int32_t* boundaries,
                             int32_t* boundary_lens, int null_slot, hipStream_t stream) {
  const int blocks = (batch + 255) / 256;
  hipLaunchKernelGGL(flush_plan_kernel, dim3(blocks), dim3(256), 0, stream, batch,
                     spec_query_len, state_indices, record_rows, pending, commit_lens,
                     final_indices, boundaries, boundary_lens, null_slot);
  return hipGetLastError();
}

}  // namespace kda
