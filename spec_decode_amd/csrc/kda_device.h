// Device helpers and internal launch interfaces of libkda (gfx950 only).
#pragma once

#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int K = 128;  // key channels per head
constexpr int V = 128;  // value channels per head
constexpr int PAGE = K * V;
constexpr int MAX_T = 8;  // largest verify window / record capacity
constexpr int WAVE = 64;

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- page stores

// Cache-policy bits of gfx950 vector memory instructions.
constexpr int CPOL_NT = 2;    // no reuse expected
constexpr int CPOL_SC1 = 16;  // device scope: a store writes through the XCD's L2
constexpr int BUF_DWORD3 = 0x00020000;  // gfx9 buffer descriptor word 3: 32-bit data format

// The MI355X memory-side cache (MALL). Launches whose state pages exceed it
// gain nothing from keeping written pages in the caches: their page accesses
// stream (write-through, no-reuse page stores; the commit also loads its pages
// with the no-reuse hint), at two workgroups per CU.
constexpr int64_t MALL_BYTES = int64_t(256) << 20;
inline bool stream_pages(int64_t page_bytes) { return page_bytes > MALL_BYTES; }

// Dynamic LDS that holds a kernel to at most two workgroups per CU (160 KiB of
// LDS per CU): the streaming instances move their pages faster with two than
// with three or more. Computed from the kernel's static LDS.
template <typename Kernel>
size_t two_per_cu_lds(Kernel kernel) {
  hipFuncAttributes a{};
  if (hipFuncGetAttributes(&a, reinterpret_cast<const void*>(kernel)) != hipSuccess) return 0;
  constexpr size_t LDS_PER_CU = 160 * 1024;
  constexpr size_t WANT = LDS_PER_CU / 3 + 256;  // three no longer fit, two do
  return a.sharedSizeBytes >= WANT ? 0 : WANT - a.sharedSizeBytes;
}

// Buffer descriptor of one page (the base must be uniform over the wave).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(void* page, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(page, 0, (int)bytes, BUF_DWORD3);
}
template <int CPOL>
__device__ __forceinline__ void store_page16(u32x4 v, __amdgpu_buffer_rsrc_t page,
                                             uint32_t byte_off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, page, (int)byte_off, 0, CPOL);
}

// ---------------------------------------------------------------- page loads

// Orders one wave's LDS accesses across its lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Contiguous page loads (the streaming instances over FP32 pages).
// Wave w loads its 32 rows (16 KiB) as 16 contiguous 1 KiB pieces with the
// no-reuse hint: piece j, lane l holds row 32w + 2j + l/32, channels
// 4(l%32) .. +3. On the large decode pool this order moves 6.15-6.29 TB/s
// in place (with the tile-order write-through stores), against 5.69-5.73 for
// plain tile-order loads and 5.82-5.86 for no-reuse tile-order loads. The
// pieces then pass through a per-wave LDS area into the tile layout.
__device__ __forceinline__ void load_page_contig(const void* page, int wave, int lane,
                                                 u32x4 (&cont)[16]) {
  const __amdgpu_buffer_rsrc_t rs = page_rsrc(const_cast<void*>(page), PAGE * 4);
#pragma unroll
  for (int j = 0; j < 16; ++j)
    cont[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, ((32 * wave + 2 * j) * K) * 4 + lane * 16,
                                                    0, CPOL_NT);
}

// The contiguous pieces into the tile layout (lane l of tile (r, cb): row
// 32w + 16r + l%16, channels 16cb + 4(l/16) .. +3), 16 rows at a time through
// the wave's LDS area of 16 rows x 32 chunks of 16 bytes. Chunk g of local row
// rho sits at slot g ^ rho of that row, so that neither the row-wise writes
// nor the column-wise tile reads meet two lanes on one bank group within a
// group of 16 lanes.
__device__ __forceinline__ void transpose_page(const u32x4 (&cont)[16], u32x4* area, int lane,
                                               u32x4 (&st)[2][8]) {
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rho = 2 * i + (lane >> 5), g = lane & 31;
      area[rho * 32 + (g ^ rho)] = cont[8 * r + i];
    }
    wave_lds_sync();
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int rho = lane & 15, g = 4 * cb + (lane >> 4);
      st[r][cb] = area[rho * 32 + (g ^ rho)];
    }
    wave_lds_sync();
  }
}

// The FP32 page in two halves (the streaming instances over FP32 pages).
// Rows 0..15 of wave w's 32 go straight into the wave's LDS area (buffer loads
// to LDS, no-reuse hint; each 1 KiB piece j lands at area + 1 KiB * j, lane l
// at byte 16 l of it): lane l of piece j fetches row 32w + rho, rho = 2j +
// l/32, the chunk g = (l % 32) ^ rho whose slot in the swizzled layout of
// transpose_page is l % 32, so each piece is still 1 KiB of contiguous page.
// Rows 16..31 load into registers as contiguous pieces (cont[i]: row
// 32w + 16 + 2i + l/32, channels 4(l % 32) .. +3). On the large decode pool
// this moves 6.32-6.36 TB/s in place against 6.11-6.12 for both halves through
// registers (same session); the whole page straight into LDS (6.32-6.42)
// would need 64 KiB of LDS per workgroup.
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void load_page_halves(const void* page, int wave, int lane,
                                                 u32x4* area, u32x4 (&cont)[8]) {
  const __amdgpu_buffer_rsrc_t rs = page_rsrc(const_cast<void*>(page), PAGE * 4);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int rho = 2 * j + (lane >> 5);
    const int g = (lane & 31) ^ rho;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(area + 64 * j), 16,
                                             ((32 * wave + rho) * K) * 4 + g * 16, 0, 0, CPOL_NT);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    cont[i] = __builtin_amdgcn_raw_buffer_load_b128(
        rs, ((32 * wave + 16 + 2 * i) * K) * 4 + lane * 16, 0, CPOL_NT);
}

// Both halves into the tile layout: wait for every load of the wave (the LDS
// half is not tracked by the compiler), read tiles (0, cb) from the area, then
// pass the register half through the same area into tiles (1, cb).
__device__ __forceinline__ void transpose_page_halves(const u32x4 (&cont)[8], u32x4* area,
                                                      int lane, u32x4 (&st)[2][8]) {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) (gfx9 encoding; expcnt, lgkmcnt not waited)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    const int rho = lane & 15, g = 4 * cb + (lane >> 4);
    st[0][cb] = area[rho * 32 + (g ^ rho)];
  }
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rho = 2 * i + (lane >> 5), g = lane & 31;
    area[rho * 32 + (g ^ rho)] = cont[i];
  }
  wave_lds_sync();
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    const int rho = lane & 15, g = 4 * cb + (lane >> 4);
    st[1][cb] = area[rho * 32 + (g ^ rho)];
  }
  wave_lds_sync();
}

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// FP32 -> BF16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __hip_bfloat16 h = __float2bfloat16(x);
  return *reinterpret_cast<uint16_t*>(&h);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------- gate math

// The bounded KDA gate decay exp(lb * sigmoid(e^{A_log} (g + dt_bias))), with
// e^{A_log} passed in precomputed. FP32 with the hardware exp2-based exp and
// reciprocal; a large negative logit gives 1 + inf -> reciprocal 0 -> d = 1.
__device__ __forceinline__ float gate_decay(float g, float exp_a_log, float dt_bias, float lb) {
  const float z = exp_a_log * (g + dt_bias);
  const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
  return __expf(lb * sig);
}

__device__ __forceinline__ float sigmoidf_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// ---------------------------------------------------------------- cross-lane

// DPP move of a float (gfx9 controls): lanes whose source is outside the
// pattern, or whose row is masked off, read 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, true));
}
constexpr int DPP_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_ROW_SHR1 = 0x111;
constexpr int DPP_ROW_SHR2 = 0x112;
constexpr int DPP_ROW_SHR4 = 0x114;
constexpr int DPP_ROW_SHR8 = 0x118;
constexpr int DPP_ROW_BCAST15 = 0x142;
constexpr int DPP_ROW_BCAST31 = 0x143;

// Sum over the 64 lanes of a wave, returned to every lane (as a scalar).
// Row sums by row shifts, then the row-broadcast steps fold the four rows into
// lane 63; no LDS round trip.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<DPP_ROW_SHR1>(x);
  x += dpp_f<DPP_ROW_SHR2>(x);
  x += dpp_f<DPP_ROW_SHR4>(x);
  x += dpp_f<DPP_ROW_SHR8>(x);
  x += dpp_f<DPP_ROW_BCAST15, 0xa>(x);
  x += dpp_f<DPP_ROW_BCAST31, 0xc>(x);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Per-lane choice by a constant lane mask: lanes whose bit is set in MASK take
// `if_set`. Written as one opaque v_cndmask so the compiler cannot turn a pair
// of such choices over one register array into a dynamically indexed read.
template <uint64_t MASK>
__device__ __forceinline__ float lane_pick(float if_set, float if_clear) {
  float r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(if_clear), "v"(if_set), "s"(MASK));
  return r;
}
constexpr uint64_t LANES_BIT0 = 0xAAAAAAAAAAAAAAAAull;  // lanes with bit 0 set
constexpr uint64_t LANES_BIT1 = 0xCCCCCCCCCCCCCCCCull;  // lanes with bit 1 set

// One transposing exchange step over lane pairs (l, l ^ DIST), DIST in {1, 2},
// on the first NV values of x: a lane keeps the half selected by its lane bit
// and adds the partner's copy of that half, halving the values it holds.
template <int NV, int DIST, int N>
__device__ __forceinline__ void quad_transpose_step(float (&x)[N]) {
  static_assert(NV <= N && NV % 2 == 0, "step over the first NV values");
  constexpr int half = NV / 2;
  constexpr uint64_t mask = DIST == 1 ? LANES_BIT0 : LANES_BIT1;
  constexpr int ctrl = DIST == 1 ? DPP_XOR1 : DPP_XOR2;
#pragma unroll
  for (int i = 0; i < half; ++i) {
    const float keep = lane_pick<mask>(x[i + half], x[i]);
    const float send = lane_pick<mask>(x[i], x[i + half]);
    x[i] = keep + dpp_f<ctrl>(send);
  }
}

// ---------------------------------------------------------------- launch params

constexpr int COMMIT_LAYERS_PER_LAUNCH = 16;

struct CommitLayer {
  void* state;            // pool base [slots][H][V][K] (BF16 bits or FP32)
  const float* corr;      // corrections [rows][H][Q][V]
  const uint16_t* kg;     // key/gate records [rows][H][Q][2K]
  int64_t state_stride;   // elements between slots
  int64_t corr_stride;    // elements between record rows
  int64_t kg_stride;      // elements between record rows
};

struct CommitParams {
  CommitLayer layer[COMMIT_LAYERS_PER_LAUNCH];
  const float* a_log;     // [L][H], at the launch's first layer
  const float* dt_bias;   // [L][H][K], at the launch's first layer
  const int32_t* sources;
  const int32_t* lens;
  const int32_t* dests;
  const int32_t* bounds;  // NULL: align off
  const int32_t* blens;
  const int32_t* rows;    // NULL: row b
  int heads;
  int null_slot;
  float lb;
};

struct VerifyParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* rb;
  const float* a_log;
  const float* dt_bias;
  void* state;             // pool base [slots][H][V][K], FP32 or BF16 bits
  int64_t slot_stride;     // elements between slots
  const int32_t* slots;
  const int32_t* rows;     // NULL (verify only): row b
  const int32_t* pending;  // fused only
  const int32_t* qsl;      // NULL: request b's rows b*T..; else [B+1] token offsets
  const int32_t* bounds;   // fused, optional (align): boundary slots [B]
  const int32_t* blens;    //   boundary lengths m [B]
  float* corr;
  uint16_t* kg;
  uint16_t* out;
  const uint16_t* gate;    // optional gated RMSNorm output stage: [B*T][H*V] BF16
  const float* norm_w;     // [V] FP32 (with gate)
  float norm_eps;
  // Optional convolution prologue (fused only; x != NULL): q, k, v computed from
  // x, replacing the q, k, v inputs.
  const uint16_t* x;       // [B*T] rows of x_stride elements: q | k | v parts of H*K
  const uint16_t* conv_w;  // [3][4][H*K] BF16
  const uint16_t* conv_b;  // [3*H*K] BF16 or NULL
  uint16_t* conv;          // window pool, element slot*conv_ss + channel*conv_cs + i*conv_ts
  int64_t x_stride;
  int64_t conv_ss, conv_cs, conv_ts;
  float q_scale;
  int rq;
  int heads;
  int null_slot;
  float lb;
};

hipError_t launch_decay(const uint16_t* raw_g, int64_t tokens, int heads, const float* a_log,
                        const float* dt_bias, float lb, float* out, hipStream_t stream);
hipError_t launch_commit(const CommitParams& p, int window, bool bf16, bool align, int batch,
                         int layers, hipStream_t stream);
hipError_t launch_verify(const VerifyParams& p, int tokens, bool fused, bool bf16, int batch,
                         hipStream_t stream);
hipError_t launch_verify_conv(const VerifyParams& p, int tokens, bool bf16, int batch,
                              hipStream_t stream);
hipError_t launch_verify_conv_packed(const VerifyParams& p, int tokens, bool bf16, int batch,
                                     hipStream_t stream);
hipError_t launch_verify_conv_window_major(const VerifyParams& p, int tokens, bool bf16,
                                           int batch, hipStream_t stream);
hipError_t launch_gate_projection(const uint16_t* f_a, int64_t sa, const uint16_t* f_b,
                                  uint16_t* out, int64_t tokens, int heads, hipStream_t stream);
hipError_t launch_page_rw(float* state, int64_t slot_stride, const int32_t* slots, int batch,
                          int heads, int null_slot, hipStream_t stream);
hipError_t launch_defer(int batch, const int32_t* state_indices, int32_t* commit_lens,
                        const int32_t* record_rows, int32_t* pending, const int32_t* eager,
                        int null_slot, hipStream_t stream);
hipError_t launch_flush_plan(int batch, int spec_query_len, const int32_t* state_indices,
                             const int32_t* record_rows, const int32_t* pending,
                             int32_t* commit_lens, int32_t* final_indices, int32_t* boundaries,
                             int32_t* boundary_lens, int null_slot, hipStream_t stream);

}  // namespace kda
