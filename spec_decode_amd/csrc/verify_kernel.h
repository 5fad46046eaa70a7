// The verify kernel template: fused replay+verify and the stock verify over
// FP32 or BF16 state pages, with the optional convolution prologue and gated
// RMSNorm output stage. Instantiated by fused.hip, fused_conv.hip,
// fused_conv_packed.hip and fused_conv_window_major.hip.
//
// Method (the vLLM page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.
// kda.fused", module docstring and KdaFused): per (request, head) item,
//  1. replay the n pending tokens from the old records in the commit's closed
//     form, S_n = S_0 diag(D_n) + sum_{t<n} u_t (kn_t * P_t)^T, writing S_n back
//     when n > 0 (the stock verify, on the page "vllm.models.kimi_k3.nvidia.
//     specialized_decode.recoverssm.kernels", is this kernel with no replay);
//  2. verify the window's T tokens from S_n in chunked (WY) form:
//     w_t = S_n (Gamma_t * kn_t), y_t = S_n (Gamma_t * q_t) (2T dots per row),
//     A_ts, B_ts pair products, then per state row
//     u_t = beta_t (v_t - w_t - sum_{s<t} A_ts u_s), o_t = y_t + sum_{s<=t} B_ts u_s;
//  3. rewrite the item's records (u_t, raw key, raw gate), after every old
//     record of the item was read.
//
// gfx950 mapping. One workgroup of 256 threads (4 wave64) per item. The page is
// held in VGPRs as 16x16 tiles, wave w owning row blocks 2w and 2w+1 (all 8
// column blocks each, 64 VGPRs). Within a tile (rows 16rb.., columns 16cb..),
// lane l holds S[16rb + l%16][16cb + 4(l/16) + i], i = 0..3: one 16-byte load
// per tile, and exactly the accumulator layout of V_MFMA_F32_16X16X4_F32 for
// the transposed tile S^T (M = key channel, N = state row). So
//  - the replay is S^T <- diag(D_n) S^T + KP U^T: 4 multiplies and one or two
//    MFMAs (K = replayed tokens, zero-padded to 4 or 8) per tile, in place;
//  - the same registers are the B operand of the dots: D2[j][v] += X[j][c] S[v][c]
//    with M = j (2T <= 16 rows of X, zero above 2T), N = v, and the 4 values of a
//    lane as 4 consecutive K steps (key channels 16cb + 4(l/16) + i);
// so no lane ever exchanges state values and every state byte is read once.
// S_n replaces the loaded page in the same registers and is stored from them
// as the kernel's last instructions. With the template argument STREAM (launches
// whose pages exceed the MALL) the window's inputs and the old records load
// with the no-reuse hint; o and the records (the stock verify), or S_n, o and
// the records (the fused step over FP32 pools, then at two workgroups per CU)
// write through the L2 with the no-reuse hint; and FP32 pages load as
// contiguous 1 KiB pieces per wave instruction (no-reuse hint), which each
// wave turns into its tiles through an LDS area of its own (transpose_page).
//
// BF16 pages hold the same register layout after conversion, with the key
// channels permuted inside each group of 32: one 16-byte load brings 8 channels
// of a row, 32j + 8(l/16) .. +7, whose first 4 serve as tile 2j and last 4 as
// tile 2j+1. A channel permutation leaves every contraction over channels
// unchanged, so only the LDS reads of X, kp and D_n follow it (chan0 below).
// S_n is stored rounded to nearest even; the verify continues from the FP32
// value, before that rounding.
//
// Convolution prologue (fused page, KdaFused.kernel; template argument CONV, 0
// without it, 1 for window pools of any strides, 2 for packed dim-first pools
// whose per-wave window blocks move as 16-byte chunks through LDS, 3 for
// window-major pools whose taps, inputs and new entries move as 16-byte
// chunks through a per-wave LDS stage): q, k
// and v are computed in the kernel from a packed row x of pre-activations, each
// channel's 4-tap causal convolution over its window in the conv pool followed
// by SiLU. The window holds the previous step's [2 history values, its T
// inputs]; after n accepted tokens the 3 taps start at max(n - 1, 0). The SiLU
// output is rounded to BF16 and is the value used everywhere (the recorded key
// is its bit pattern), so that rounding is taken by fixed FP32 steps: an fma
// chain in tap order from the bias, exp by a Cody-Waite reduction and a degree-7
// Taylor polynomial, an IEEE divide, round to nearest even. q is then
// L2-normalised (1e-6 inside the root) and scaled by q_scale; the window is
// rewritten as [tap 1, tap 2, x_0 .. x_{T-1}]. Threads 0..127 convolve the q and
// k parts of channel c, threads 128..255 the v part.
//
// Prologue (while the page loads are in flight): threads 0..127 (channel c) do
// the new tokens (decays, key norms, Gamma, X, the T^2 pair products reduced
// over channels by a transposing wave reduction); threads 128..255 do the old
// records (decays, norms, kp_t = kn_t * prod_{t<s<n} d_s, D_n), the
// corrections, v and beta. Loads return in order, so threads 0..127 issue their
// small loads before the page and start the prologue while it streams in;
// threads 128..255 issue the page first (their records are needed later), with
// the convolution's v operands ahead of it.
#pragma once

#include <type_traits>
#include <utility>

#include "kda_device.h"

// A measurement variant, never built by default: with -DKDA_VALU_DOTS=1 the
// instances over FP32 pages form the 2T row dots ([V x K] x [K x 2T] per item)
// with plain FP32 FMAs instead of MFMA: after the state pass, one dot column
// at a time, each lane sums its 32 channels of its two rows from the page
// registers and the row's four lane groups add their sums by lane exchanges
// (the replay keeps its MFMAs). It exists to time the MFMA choice for this
// product against the vector ALU on the same kernel.
#ifndef KDA_VALU_DOTS
#define KDA_VALU_DOTS 0
#endif

namespace kda {

constexpr bool kValuDots = KDA_VALU_DOTS != 0;

template <int T>
struct Pairs {
  static constexpr int NA = T * (T - 1) / 2;  // A_ts, s < t
  static constexpr int NP = T * T;            // then B_ts, s <= t
  static constexpr int P2 = NP <= 1 ? 1 : NP <= 2 ? 2 : NP <= 4 ? 4 : NP <= 8 ? 8
                          : NP <= 16 ? 16 : NP <= 32 ? 32 : 64;
  __device__ static constexpr int a(int t, int s) { return t * (t - 1) / 2 + s; }
  __device__ static constexpr int b(int t, int s) { return NA + t * (t + 1) / 2 + s; }
};

// Which pair product sits at index i: A_ts (s < t) at t(t-1)/2 + s, then B_ts
// (s <= t) at NA + t(t+1)/2 + s. Built at compile time so that every register
// index below folds to a constant.
template <int T>
struct PairTable {
  int s[64], t[64], is_a[64];
  constexpr PairTable() : s(), t(), is_a() {
    int i = 0;
    for (int tt = 1; tt < T; ++tt)
      for (int ss = 0; ss < tt; ++ss) { s[i] = ss; t[i] = tt; is_a[i] = 1; ++i; }
    for (int tt = 0; tt < T; ++tt)
      for (int ss = 0; ss <= tt; ++ss) { s[i] = ss; t[i] = tt; is_a[i] = 0; ++i; }
    for (; i < 64; ++i) { s[i] = 0; t[i] = 0; is_a[i] = -1; }
  }
};

// This channel's share of pair product I: A_ts = kn_s * P(s,t) * kn_t or
// B_ts = kn_s * P(s,t) * q_t with P(s,t) = prod_{s<r<=t} d_r; zero past T^2.
template <int T, int I>
__device__ __forceinline__ float pair_share(const float (&kn)[T], const float (&q)[T],
                                            const float (&d)[T]) {
  constexpr PairTable<T> tab{};
  constexpr int s = tab.s[I], t = tab.t[I], kind = tab.is_a[I];
  if constexpr (kind < 0) {
    return 0.f;
  } else {
    float pr = kn[s];
#pragma unroll
    for (int r = s + 1; r <= t; ++r) pr *= d[r];
    return pr * (kind == 1 ? kn[t] : q[t]);
  }
}

// Pair products I and I + HALF folded by the first transposing step (lane pairs
// l, l ^ 1): the lane keeps the one its bit 0 selects and adds its partner's
// copy of it. Forming each pair just before it is folded keeps only HALF
// partial sums live instead of all the products.
template <int T, int HALF, int I>
__device__ __forceinline__ float pair_fold_first(const float (&kn)[T], const float (&q)[T],
                                                 const float (&d)[T]) {
  const float lo = pair_share<T, I>(kn, q, d);
  const float hi = pair_share<T, I + HALF>(kn, q, d);
  const float keep = lane_pick<LANES_BIT0>(hi, lo);
  const float send = lane_pick<LANES_BIT0>(lo, hi);
  return keep + dpp_f<DPP_XOR1>(send);
}

// The pair products summed over the 128 channels, stage one (lower waves, one
// channel per lane): two in-register transposing steps over the lane quads
// leave each lane P2/4 partial sums of 4 channels (for P2 >= 4), which go to
// part[pair][quad of the half] in LDS; stage two sums those per pair.
template <int T>
struct PairStage {
  static constexpr int P2 = Pairs<T>::P2;
  static constexpr int STEPS = P2 >= 4 ? 2 : (P2 == 2 ? 1 : 0);
  static constexpr int R = P2 >> STEPS;           // values a lane keeps
  static constexpr int PARTS = 128 >> STEPS;      // partials per pair (both waves)
};

// Is: 0 .. P2/2 - 1 (one fold per index) when there is a step, else just 0.
template <int T, int... Is>
__device__ __forceinline__ void pair_stage_one(const float (&kn)[T], const float (&q)[T],
                                               const float (&d)[T], int lane, int wave,
                                               float* part, std::integer_sequence<int, Is...>) {
  using PS = PairStage<T>;
  float pv[PS::P2];
  if constexpr (PS::STEPS >= 1) {
    ((pv[Is] = pair_fold_first<T, PS::P2 / 2, Is>(kn, q, d)), ...);
    if constexpr (PS::STEPS >= 2) quad_transpose_step<PS::P2 / 2, 2>(pv);
  } else {
    pv[0] = pair_share<T, 0>(kn, q, d);
  }
  // Lane l now holds, in slot i, pair i + R*(bit1 of l) + 2R*(bit0 of l)
  // (only the bits the steps used), summed over its 2^STEPS lanes.
  const int sel = PS::STEPS == 2 ? ((lane & 1) * 2 + ((lane >> 1) & 1))
                  : (PS::STEPS == 1 ? (lane & 1) : 0);
  const int group = wave * (64 >> PS::STEPS) + (lane >> PS::STEPS);
#pragma unroll
  for (int i = 0; i < PS::R; ++i) part[(i + PS::R * sel) * PS::PARTS + group] = pv[i];
}

// exp in FP32 for the convolution's SiLU: x clamped to [-80, 80],
// k = rint(x log2 e), r = x - k ln2 by two fmas (ln2 split into its value
// rounded to 16 fraction bits and the FP32 remainder), then the Taylor
// polynomial sum_{j<=7} r^j / j! in Horner form (fma), scaled by 2^k.
__device__ __forceinline__ float conv_exp(float x) {
  constexpr float kLn2Hi = 45426.0f / 65536.0f;
  constexpr float kLn2Lo = (float)(0.69314718055994530942 - (double)kLn2Hi);
  constexpr float kLog2e = 1.44269504088896340736f;
  x = fminf(fmaxf(x, -80.0f), 80.0f);
  const float k = rintf(x * kLog2e);
  float r = __builtin_fmaf(-k, kLn2Hi, x);
  r = __builtin_fmaf(-k, kLn2Lo, r);
  float p = 1.0f / 5040.0f;                 // 1/7!
  p = __builtin_fmaf(p, r, 1.0f / 720.0f);  // 1/6!
  p = __builtin_fmaf(p, r, 1.0f / 120.0f);
  p = __builtin_fmaf(p, r, 1.0f / 24.0f);
  p = __builtin_fmaf(p, r, 1.0f / 6.0f);
  p = __builtin_fmaf(p, r, 1.0f / 2.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return ldexpf(p, (int)k);
}

// One channel's convolution outputs: seq = 3 taps then T inputs, w the 4
// weights (w[3] meets the current input). Returns the BF16 bits of SiLU.
template <int T>
__device__ __forceinline__ void conv_silu(const float (&seq)[3 + T], const float (&w)[4],
                                          float bias, uint32_t (&y)[T]) {
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float acc = bias;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(seq[t + i], w[i], acc);
    const float e = conv_exp(-acc);
    y[t] = f32_to_bf16_bits(__fdiv_rn(acc, 1.0f + e));
  }
}

// Window pool layouts of the convolution prologue: any strides, or packed
// dim-first windows (tap stride 1, channel stride W = RQ + 2, slot stride a
// multiple of 8 elements, 16-byte aligned base). In the packed layout the
// windows of a wave's 64 channels are one contiguous block of 128 W bytes,
// which the wave moves with 16-byte accesses through LDS.
constexpr int CONV_NONE = 0, CONV_STRIDED = 1, CONV_PACKED = 2, CONV_WINDOW_MAJOR = 3;
constexpr int CONV_BLOCK = 64 * (MAX_T + 2) * 2;  // LDS bytes of one wave's block, W <= MAX_T + 2
// Window-major pools (channel stride 1, tap and slot strides and the input
// rows 16-byte aligned): a wave stages its 64 channels' 3 taps and T inputs as
// rows of 128 bytes, [tap 0, tap 1, tap 2, x_0 .. x_{T-1}], moved in and out
// with 16-byte accesses. The new window [tap 1, tap 2, x_0 .. x_{T-1}] is rows
// 1 .. T + 2 of the stage.
constexpr int CONV_STAGE = 64 * (MAX_T + 3) * 2;  // LDS bytes of one wave's stage
template <int MODE>
constexpr int conv_area() { return MODE == CONV_WINDOW_MAJOR ? CONV_STAGE : CONV_BLOCK; }

// One channel's convolution operands as raw BF16 bits: the T inputs, the 4
// weights and the bias; strided layout: the 3 window taps at the item's
// offset; packed layout: the wave's window block, 16-byte chunks lane and
// lane + 64 (clamped to the last chunk); window-major layout: instead of the
// inputs and taps, the lane's 16-byte chunk of the wave's input rows (row
// lane / 8, channels 8 (lane % 8) .. +7) and of its tap rows.
template <int T>
struct ConvIn {
  uint32_t tap[3];
  u32x4 blk[2];
  uint32_t x[T];
  u32x4 xv, tv;
  uint32_t w[4];
  uint32_t bias;
};

// Loads of channel col (= part * H*K + head channel) of the conv operands. The
// taps start at the wave-uniform offset off = max(n - 1, 0) <= RQ - 1, so the
// last one, off + 2 <= RQ + 1, lies inside the window of RQ + 2 entries. The
// inputs, weights and bias do not depend on n and are issued first.
template <int T, int MODE, bool NT = false>
__device__ __forceinline__ void conv_load(const VerifyParams& p, ConvIn<T>& ci, int slot,
                                          int64_t col, int64_t head_row, int part,
                                          int64_t dim, int64_t tok0, int off) {
  const int lane = threadIdx.x & (WAVE - 1);
  if constexpr (MODE == CONV_WINDOW_MAJOR) {
    // Row lane / 8 (clamped: lanes past the last row load it again), channels
    // 8 (lane % 8) .. +7 of the wave's 64 (col - lane .. col - lane + 63).
    const int r = lane >> 3;
    const int64_t ch = col - lane + 8 * (lane & 7);
    const u32x4* const xp =
        reinterpret_cast<const u32x4*>(p.x + (tok0 + (r < T ? r : T - 1)) * p.x_stride + ch);
    ci.xv = NT ? __builtin_nontemporal_load(xp) : *xp;
  } else {
#pragma unroll
    for (int t = 0; t < T; ++t) ci.x[t] = p.x[(tok0 + t) * p.x_stride + col];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) ci.w[i] = p.conv_w[(part * 4 + i) * dim + head_row];
  // Unconditional (without a bias, from the weights, col < 3HK <= 12HK, then
  // dropped): a load under a branch ends in a wait for every load before it.
  const bool has_bias = p.conv_b != nullptr;
  const uint32_t braw = (has_bias ? p.conv_b : p.conv_w)[col];
  ci.bias = has_bias ? braw : 0u;
  if constexpr (MODE == CONV_WINDOW_MAJOR) {
    // Tap row off + lane / 8 (lanes 0..23; the others load the last one again).
    const int r = lane >> 3;
    const int64_t ch = col - lane + 8 * (lane & 7);
    const u32x4* const tp = reinterpret_cast<const u32x4*>(
        p.conv + (int64_t)slot * p.conv_ss + (int64_t)(off + (r < 3 ? r : 2)) * p.conv_ts + ch);
    ci.tv = NT ? __builtin_nontemporal_load(tp) : *tp;
  } else if constexpr (MODE == CONV_PACKED) {
    // The block of channels col0 .. col0 + 63 (col0 = col rounded down to 64:
    // a wave's channels), 8 W chunks of 16 bytes.
    const int W = p.rq + 2;
    const int nchunk = 8 * W;
    const u32x4* bp = reinterpret_cast<const u32x4*>(
        p.conv + (int64_t)slot * p.conv_ss + (col & ~(int64_t)63) * W);
    ci.blk[0] = bp[lane < nchunk ? lane : nchunk - 1];
    ci.blk[1] = bp[lane + WAVE < nchunk ? lane + WAVE : nchunk - 1];
  } else {
    const uint16_t* wp = p.conv + (int64_t)slot * p.conv_ss + col * p.conv_cs;
#pragma unroll
    for (int i = 0; i < 3; ++i) ci.tap[i] = wp[(int64_t)(off + i) * p.conv_ts];
  }
}


// The window write-back [tap 1, tap 2, x_0 .. x_{T-1}] (entries past T + 1 keep
// their values; the thread rewrites only entries of its own channel), then the
// channel's convolution + SiLU (BF16 bits into y). Storing first lets the raw
// bits die as they are converted. Packed layout: the block goes to the wave's
// LDS area blk_s (CONV_BLOCK bytes), each lane reads its taps there and writes
// its new entries back, and the wave stores the whole block.
template <int T, int MODE, bool NT = false>
__device__ __forceinline__ void conv_part(const VerifyParams& p, const ConvIn<T>& ci, int slot,
                                          int64_t col, int off, uint8_t* blk_s,
                                          uint32_t (&y)[T]) {
  uint32_t tap[3];
  uint32_t xin[T];
  if constexpr (MODE == CONV_WINDOW_MAJOR) {
    // Stage rows [tap 0..2, x_0 .. x_{T-1}] of 8 chunks each, read the lane's
    // channel back, then store rows 1 .. T + 2 as window entries 0 .. T + 1.
    const int lane = threadIdx.x & (WAVE - 1);
    u32x4* const sv = reinterpret_cast<u32x4*>(blk_s);
    const uint16_t* const sh = reinterpret_cast<const uint16_t*>(blk_s);
    if (lane < 24) sv[lane] = ci.tv;
    if (lane < 8 * T) sv[24 + lane] = ci.xv;
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 3; ++i) tap[i] = sh[i * 64 + lane];
#pragma unroll
    for (int t = 0; t < T; ++t) xin[t] = sh[(3 + t) * 64 + lane];
    uint16_t* const wp = p.conv + (int64_t)slot * p.conv_ss + (col - lane);
    constexpr int NCH = 8 * (T + 2);
#pragma unroll
    for (int q0 = 0; q0 < NCH; q0 += WAVE) {
      const int q = q0 + lane;
      if (q < NCH) {
        u32x4* const dp =
            reinterpret_cast<u32x4*>(wp + (int64_t)(q >> 3) * p.conv_ts + 8 * (q & 7));
        if constexpr (NT)
          __builtin_nontemporal_store(sv[8 + q], dp);
        else
          *dp = sv[8 + q];
      }
    }
  } else if constexpr (MODE == CONV_PACKED) {
    const int W = p.rq + 2;
    const int nchunk = 8 * W;
    const int lane = threadIdx.x & (WAVE - 1);
    u32x4* const bs = reinterpret_cast<u32x4*>(blk_s);
    if (lane < nchunk) bs[lane] = ci.blk[0];
    if (lane + WAVE < nchunk) bs[lane + WAVE] = ci.blk[1];
    wave_lds_sync();
    uint16_t* const mine = reinterpret_cast<uint16_t*>(blk_s) + (col & 63) * W;
#pragma unroll
    for (int i = 0; i < 3; ++i) tap[i] = mine[off + i];
    mine[0] = (uint16_t)tap[1];
    mine[1] = (uint16_t)tap[2];
#pragma unroll
    for (int t = 0; t < T; ++t) mine[2 + t] = (uint16_t)ci.x[t];
#pragma unroll
    for (int t = 0; t < T; ++t) xin[t] = ci.x[t];
    wave_lds_sync();
    u32x4* const bp = reinterpret_cast<u32x4*>(
        p.conv + (int64_t)slot * p.conv_ss + (col & ~(int64_t)63) * W);
    if (lane < nchunk) bp[lane] = bs[lane];
    if (lane + WAVE < nchunk) bp[lane + WAVE] = bs[lane + WAVE];
  } else {
#pragma unroll
    for (int i = 0; i < 3; ++i) tap[i] = ci.tap[i];
    uint16_t* wp = p.conv + (int64_t)slot * p.conv_ss + col * p.conv_cs;
    wp[0] = (uint16_t)tap[1];
    wp[p.conv_ts] = (uint16_t)tap[2];
#pragma unroll
    for (int t = 0; t < T; ++t) wp[(int64_t)(2 + t) * p.conv_ts] = (uint16_t)ci.x[t];
#pragma unroll
    for (int t = 0; t < T; ++t) xin[t] = ci.x[t];
  }
  float seq[3 + T];
  float w[4];
#pragma unroll
  for (int i = 0; i < 3; ++i) seq[i] = bf16_bits_to_f32(tap[i]);
#pragma unroll
  for (int t = 0; t < T; ++t) seq[3 + t] = bf16_bits_to_f32(xin[t]);
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = bf16_bits_to_f32(ci.w[i]);
  conv_silu<T>(seq, w, bf16_bits_to_f32(ci.bias), y);
}

// First key channel of lane group g (= lane / 16) in tile cb: values i = 0..3
// of the lane are channels chan0 + i.
template <bool SB16>
__device__ __forceinline__ constexpr int chan0(int cb, int g) {
  return SB16 ? 32 * (cb >> 1) + 8 * g + 4 * (cb & 1) : 16 * cb + 4 * g;
}

template <int T, bool FUSED, bool GATED, bool SB16, int CONV, bool STREAM = false>
__global__ __launch_bounds__(256) void verify_kernel(const VerifyParams p) {
  static_assert(FUSED || !CONV, "the convolution prologue is a fused-step prologue");
  // Write-through stores (STREAM): the stock verify's o and records, and the
  // fused step's S_n, o and records, on either pool.
  constexpr bool kWriteThrough = STREAM;
  // Contiguous no-reuse page loads through an LDS transpose: the streaming
  // instances over FP32 pages (fused step 0.812 -> 0.785 ms, stock verify
  // 0.507 -> 0.487 ms on the large decode batch).
  constexpr bool kContig = STREAM && !SB16;
  using PI = Pairs<T>;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int H = p.heads;
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  // The wave index as a scalar: branches on it are uniform (s_cbranch), so a
  // wave runs only its own half's code and waits only on its own loads.
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  // The item's window: rows tok0 .. tok0 + L - 1. With query_start_loc the
  // length is qsl[b+1] - qsl[b], clamped to 0..T; an empty window is padding
  // and nothing is read or written. Tokens t >= L are masked below (zero key,
  // q, v and beta), which leaves every result of the tokens t < L unchanged.
  int64_t tok0 = (int64_t)b * T;
  int L = T;
  if (p.qsl != nullptr) {
    const int q0 = __builtin_amdgcn_readfirstlane(p.qsl[b]);
    const int q1 = __builtin_amdgcn_readfirstlane(p.qsl[b + 1]);
    tok0 = q0;
    L = q1 - q0;
    L = L < 0 ? 0 : (L > T ? T : L);
    if (L == 0) return;
  }
  const int last = L - 1;  // rows past the window read the last token (then masked)

  const int slot = p.slots[b];
  if (slot <= p.null_slot) {
    // No state: the item's outputs are zero and nothing else is written.
    if (tid < L * (V / 8)) {
      const int t = tid / (V / 8);
      const int c = (tid % (V / 8)) * 8;
      *reinterpret_cast<uint4*>(p.out + ((tok0 + t) * H + h) * V + c) = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  const int rec = p.rows != nullptr ? p.rows[b] : b;
  int n = 0;
  if constexpr (FUSED) {
    if (rec >= 0) {
      n = p.pending[rec];
      n = n < 0 ? 0 : (n > p.rq ? p.rq : n);
    }
  }
  const bool replay = FUSED && n > 0;
  // Boundary store (align, fused only): S_me, me = min(m, n), also goes to the
  // boundary slot when the replay runs, the slot is live and m > 0. The fold
  // then runs in two stages, tokens [0, me) and [me, n).
  int me = 0, bslot = 0;
  if constexpr (FUSED) {
    if (replay && p.bounds != nullptr) {
      const int bs = __builtin_amdgcn_readfirstlane(p.bounds[b]);
      const int m = __builtin_amdgcn_readfirstlane(p.blens[b]);
      if (bs > p.null_slot && m > 0) {
        me = m < n ? m : n;
        bslot = bs;
      }
    }
  }
  const bool balign = me > 0;

  // BF16 pages: LDS bounds the occupancy, so x_s (read only in the state pass)
  // and dots_s (written after it, behind a barrier) share their 8 KiB. With
  // FP32 pages they stay apart: the fused FP32 instance fits 4 workgroups per
  // CU in registers (128 VGPRs) but ran slower with them than with the 3 its
  // LDS allows.
  constexpr bool kShareXD = SB16;
  // Rows padded by 4 floats (16 bytes): the state pass reads x_s as 16-byte
  // pieces of 16 different rows per instruction, and the solve reads dots_s
  // down a column (one state row per lane); with 512-byte rows both would meet
  // every lane on the same banks.
  constexpr int XP = K + 4;
  __shared__ __attribute__((aligned(16))) float x_s[16][XP];  // Gamma_t kn_t | Gamma_t q_t | 0
  __shared__ __attribute__((aligned(16))) float dots_own[kShareXD ? 1 : 16][XP];
  float (*const dots_s)[XP] =
      kShareXD ? x_s : dots_own;  // [j][state row]: w_t (j = t) | y_t (j = T + t)
  __shared__ __attribute__((aligned(16))) float kp_s[MAX_T][K];  // replay kn_t P_t (0 past n)
  __shared__ __attribute__((aligned(16))) float u_s[MAX_T][V];   // replay u_t (0 past n)
  __shared__ __attribute__((aligned(16))) float dn_s[K];
  __shared__ __attribute__((aligned(16))) float kpm_s[MAX_T][K];  // align: stage one kn_t P_t
  __shared__ __attribute__((aligned(16))) float dm_s[K];          // align: D_me
  __shared__ __attribute__((aligned(16))) float v_s[T][V];
  __shared__ float pair_s[PI::P2];
  __shared__ __attribute__((aligned(16))) float part_s[PI::P2][PairStage<T>::PARTS];
  __shared__ float ssq_s[2][2][MAX_T];  // [new | old keys][wave of the half][token]
  __shared__ float qsq_s[2][MAX_T];     // convolution prologue: q sums of squares
  __shared__ float beta_s[MAX_T];
  __shared__ uint32_t kg_s[T][K];  // raw key | raw gate << 16 of the window, for the records
  // kContig: each wave's transpose area, 16 rows x 32 chunks of 16 bytes.
  __shared__ __attribute__((aligned(16))) u32x4 xt_s[kContig ? 4 : 1][kContig ? 16 * 32 : 1];

  const int c = tid & (K - 1);   // channel / state row of this thread's half
  const bool lower = wave < 2;   // threads 0..127: new tokens; 128..255: records, v, beta
  const int64_t head_row = (int64_t)h * K + c;

  // ---- 1-2. Loads. Loads return in order, so a wave's first use of a small
  // input waits for every load issued before it. The new-token waves (0, 1)
  // issue their small loads first and the page after, so their prologue starts
  // while the page streams in; the record waves (2, 3) issue the page first,
  // then theirs (their prologue needs the records, which arrive after).
  const float a_log_h = p.a_log[h];
  const float dtb = p.dt_bias[head_row];
  // Output stage inputs (compiled in only for the gated instances): wave w
  // finishes tokens 2w and 2w + 1, each lane rows lane and lane + 64 of them.
  float nw[2] = {1.f, 1.f};
  uint32_t gtb[2][2];
  if constexpr (GATED) {
#pragma unroll
    for (int i = 0; i < 2; ++i) nw[i] = p.norm_w[lane + 64 * i];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = 2 * wave + j;
      const int64_t row = (tok0 + (t < L ? t : last)) * H * V + (int64_t)h * V;
#pragma unroll
      for (int i = 0; i < 2; ++i) gtb[j][i] = p.gate[row + lane + 64 * i];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  uint32_t kb[T], gb[T], qb[T];  // lower: new raw key, gate, q bits
  uint32_t vb[T];                // upper: new v bits
  // Convolution prologue: per part this thread convolves (lower: q, k; upper:
  // v), the 3 taps at the replay-aware offset (after n accepted tokens they
  // start at n - 1; n = 0 reads from 0), the T inputs, the 4 weights and the
  // bias, all as raw BF16 bits.
  ConvIn<T> cin0, cin1;  // lower: q part, k part; upper: v part in cin0
  const int64_t dim = (int64_t)H * K;
  const int conv_off = n > 0 ? n - 1 : 0;
  // Packed window blocks and window-major stages go through x_s, which is
  // first written after the prologue's part one: areas 2w, 2w + 1 (q, k) of
  // lower wave w, w + 2 (v) of upper wave w, 6 areas <= sizeof x_s.
  uint8_t* const blk_s = reinterpret_cast<uint8_t*>(&x_s[0][0]);
  constexpr int CA = conv_area<CONV>();
  static_assert(6 * CA <= 16 * XP * sizeof(float), "window blocks fit in x_s");
  uint32_t okb[MAX_T], ogb[MAX_T];
  float ou[MAX_T];
  uint32_t rbb = 0;
  // Page tiles: 16-byte loads, one per tile (FP32) or per pair of tiles (BF16),
  // kept as loaded until the state pass converts them.
  constexpr int ES = SB16 ? 2 : 4;        // bytes per state element
  constexpr int NLD = SB16 ? 4 : 8;       // 16-byte loads per row block
  constexpr int LDC = 16 / ES;            // channels per load
  const int lr = lane & 15;  // row within a tile
  const int lq = lane >> 4;  // channel group within a tile
  char* const page = static_cast<char*>(p.state) +
                     ((int64_t)slot * p.slot_stride + (int64_t)h * PAGE) * ES;
  char* const tile0 = page + ((16 * (2 * wave) + lr) * K + LDC * lq) * ES;
  u32x4 st[2][NLD];
  // kContig: the page pieces as loaded into registers. The stock verify loads
  // half of each wave's share straight into the wave's LDS area instead
  // (load_page_halves; 0.480 -> 0.471 ms on the large decode batch). The fused
  // step keeps both halves in registers: with the LDS half it is slower on
  // that batch (0.784-0.786 -> 0.787-0.791 ms, gated 0.785 -> 0.797 ms), also
  // when the barrier that closes the prologue waits for LDS accesses only
  // instead of for the wave's loads into LDS too.
  constexpr bool kHalves = kContig && !FUSED;
  u32x4 cont[kContig ? 16 : 1];
  float kf[T], qf[T], dnew[T];
  float okf[MAX_T], od[MAX_T];
  // ---- 3. Prologue, part one: decays, key sums of squares, staging; with the
  // convolution, first the window write-back and the convolution + SiLU (each
  // thread touches only the window entries of its own channels). Each half's
  // loads and part one form one branch, so no merge point holds both halves'
  // loaded values at once.
  if (lower) {
    if constexpr (CONV) {
      conv_load<T, CONV, STREAM>(p, cin0, slot, 0 * dim + head_row, head_row, 0, dim, tok0,
                                 conv_off);
      conv_load<T, CONV, STREAM>(p, cin1, slot, 1 * dim + head_row, head_row, 1, dim, tok0,
                                 conv_off);
#pragma unroll
      for (int t = 0; t < T; ++t) gb[t] = p.g[(tok0 + (t < L ? t : last)) * H * K + head_row];
    } else {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int64_t idx = (tok0 + (t < L ? t : last)) * H * K + head_row;
        // STREAM: the window's inputs are read once (no-reuse hint).
        kb[t] = STREAM ? __builtin_nontemporal_load(p.k + idx) : p.k[idx];
        gb[t] = STREAM ? __builtin_nontemporal_load(p.g + idx) : p.g[idx];
        qb[t] = STREAM ? __builtin_nontemporal_load(p.q + idx) : p.q[idx];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kContig) {
      if constexpr (kHalves)
        load_page_halves(page, wave, lane, &xt_s[wave][0], reinterpret_cast<u32x4(&)[8]>(cont));
      else
        load_page_contig(page, wave, lane, cont);
    } else {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int j = 0; j < NLD; ++j)
          st[r][j] = *reinterpret_cast<const u32x4*>(tile0 + (16 * r * K + 4 * LDC * j) * ES);
    }
    __builtin_amdgcn_sched_barrier(0);
    const float ea = __expf(a_log_h);
    if constexpr (CONV) {
      conv_part<T, CONV, STREAM>(p, cin0, slot, 0 * dim + head_row, conv_off,
                                 blk_s + 2 * wave * CA, qb);
      conv_part<T, CONV, STREAM>(p, cin1, slot, 1 * dim + head_row, conv_off,
                                 blk_s + (2 * wave + 1) * CA, kb);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      kf[t] = t < L ? bf16_bits_to_f32(kb[t]) : 0.f;
      qf[t] = t < L ? bf16_bits_to_f32(qb[t]) : 0.f;
      if constexpr (CONV) {
        const float sq = wave_sum(qf[t] * qf[t]);
        if (lane == 0) qsq_s[wave][t] = sq;
      }
      dnew[t] = gate_decay(bf16_bits_to_f32(gb[t]), ea, dtb, p.lb);
      kg_s[t][c] = kb[t] | (gb[t] << 16);  // raw bits for the record write-back
      const float s = wave_sum(kf[t] * kf[t]);
      if (lane == 0) ssq_s[0][wave][t] = s;
    }
  } else {
    // The v part's convolution operands go before the page, so that its
    // convolution runs while the page streams in.
    if constexpr (CONV) {
      conv_load<T, CONV, STREAM>(p, cin0, slot, 2 * dim + head_row, head_row, 2, dim, tok0,
                                 conv_off);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kContig) {
      if constexpr (kHalves)
        load_page_halves(page, wave, lane, &xt_s[wave][0], reinterpret_cast<u32x4(&)[8]>(cont));
      else
        load_page_contig(page, wave, lane, cont);
    } else {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int j = 0; j < NLD; ++j)
          st[r][j] = *reinterpret_cast<const u32x4*>(tile0 + (16 * r * K + 4 * LDC * j) * ES);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!CONV) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int64_t idx = (tok0 + (t < L ? t : last)) * H * V + head_row;
        vb[t] = STREAM ? __builtin_nontemporal_load(p.v + idx) : p.v[idx];
      }
    }
    rbb = p.rb[(tok0 + (c < L ? c : last)) * H + h];  // unconditional: no divergent load
    if constexpr (CONV) {
      // Before the record loads: their count depends on n, so a wait placed
      // after them could not tell the convolution's operands from the page.
      __builtin_amdgcn_sched_barrier(0);
      conv_part<T, CONV, STREAM>(p, cin0, slot, 2 * dim + head_row, conv_off,
                                 blk_s + (wave + 2) * CA, vb);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (FUSED) {
      const int64_t rbase = ((int64_t)(rec < 0 ? 0 : rec) * H + h) * p.rq;
#pragma unroll
      for (int t = 0; t < MAX_T; ++t) {
        okb[t] = 0;
        ogb[t] = 0;
        ou[t] = 0.f;
        if (t < n) {
          // STREAM: the old records are read once (no-reuse hint).
          const uint16_t* const kgp = p.kg + (rbase + t) * 2 * K + c;
          const float* const up = p.corr + (rbase + t) * V + c;
          okb[t] = STREAM ? __builtin_nontemporal_load(kgp) : kgp[0];
          ogb[t] = STREAM ? __builtin_nontemporal_load(kgp + K) : kgp[K];
          ou[t] = STREAM ? __builtin_nontemporal_load(up) : up[0];
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const float ea = __expf(a_log_h);
#pragma unroll
    for (int t = 0; t < T; ++t) v_s[t][c] = t < L ? bf16_bits_to_f32(vb[t]) : 0.f;
    if (c < T) beta_s[c] = c < L ? sigmoidf_fast(bf16_bits_to_f32(rbb)) : 0.f;
    if constexpr (FUSED) {
      if (replay) {
#pragma unroll
        for (int t = 0; t < MAX_T; ++t) {
          okf[t] = bf16_bits_to_f32(okb[t]);
          od[t] = gate_decay(bf16_bits_to_f32(ogb[t]), ea, dtb, p.lb);
          u_s[t][c] = ou[t];  // zero past n
          if (t < n) {
            const float s = wave_sum(okf[t] * okf[t]);
            if (lane == 0) ssq_s[1][wave - 2][t] = s;
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- 4. Prologue, part two: X, pair products, replay coefficients.
  if (lower) {
    float kn[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
      kn[t] = kf[t] * __builtin_amdgcn_rsqf(ssq_s[0][0][t] + ssq_s[0][1][t] + 1e-6f);
    if constexpr (CONV) {
#pragma unroll
      for (int t = 0; t < T; ++t)
        qf[t] = qf[t] * __builtin_amdgcn_rsqf(qsq_s[0][t] + qsq_s[1][t] + 1e-6f) * p.q_scale;
    }
    float gam = 1.f;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      gam *= dnew[t];
      x_s[t][c] = gam * kn[t];
      x_s[T + t][c] = gam * qf[t];
    }
#pragma unroll
    for (int j = 2 * T; j < 16; ++j) x_s[j][c] = 0.f;
    // A_ts, B_ts summed over the 128 channels: two transposing steps in
    // registers (the first folds each pair as it is formed), then the two
    // waves' partial sums meet in LDS.
    pair_stage_one<T>(kn, qf, dnew, lane, wave, &part_s[0][0],
                      std::make_integer_sequence<int, (PairStage<T>::STEPS >= 1 ? PI::P2 / 2
                                                                                : 1)>{});
  } else {
    if constexpr (FUSED) {
      if (replay) {
        // The recorded keys' norms, in two halves, so that at most 8 of the 16
        // sums of squares are live next to the page.
        float knr[MAX_T];
#pragma unroll
        for (int t = 0; t < MAX_T; ++t) {
          if (t == MAX_T / 2) __builtin_amdgcn_sched_barrier(0);
          knr[t] = okf[t] * __builtin_amdgcn_rsqf(ssq_s[1][0][t] + ssq_s[1][1][t] + 1e-6f);
        }
        // Suffix products over the fold's stages: stage two (tokens me..n-1,
        // all n without align) into kp_s / dn_s, stage one (tokens 0..me-1)
        // into kpm_s / dm_s.
        float pp = 1.f;
#pragma unroll
        for (int t = MAX_T - 1; t >= 0; --t) {
          float w = 0.f;
          if (t < n && t >= me) {
            w = knr[t] * pp;
            pp *= od[t];
          }
          kp_s[t][c] = w;
        }
        dn_s[c] = pp;
        if (balign) {
          float pm = 1.f;
#pragma unroll
          for (int t = MAX_T - 1; t >= 0; --t) {
            float w = 0.f;
            if (t < me) {
              w = knr[t] * pm;
              pm *= od[t];
            }
            kpm_s[t][c] = w;
          }
          dm_s[c] = pm;
        }
      }
    }
  }
  // The contiguous pieces into the tile layout, each wave its own rows (no
  // workgroup barrier), before the barrier that the record waves reach first.
  if constexpr (kContig) {
    if constexpr (!SB16) {
      if constexpr (kHalves)
        transpose_page_halves(reinterpret_cast<const u32x4(&)[8]>(cont), &xt_s[wave][0], lane,
                              st);
      else
        transpose_page(cont, &xt_s[wave][0], lane, st);
    }
  }
  __syncthreads();

  // ---- Pair products, stage two: 4 threads per pair add its partials.
  {
    using PS = PairStage<T>;
    constexpr int PER = PS::PARTS / 4;
    if (tid < PS::P2 * 4) {
      const int pr = tid >> 2;
      const float* src = &part_s[pr][(tid & 3) * PER];
      float acc2 = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc2 += src[i];
      acc2 += dpp_f<DPP_XOR1>(acc2);
      acc2 += dpp_f<DPP_XOR2>(acc2);
      if ((tid & 3) == 0) pair_s[pr] = acc2;
    }
  }

  // ---- 5. The state pass: replay in place (MFMA), store S_n, 2T dots (MFMA).
  float ub[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  if (replay) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int vrow = 16 * (2 * wave + r) + lr;
      ub[r][0] = u_s[lq][vrow];
      ub[r][1] = u_s[4 + lq][vrow];
    }
  }
  floatx4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  constexpr bool kValu = kValuDots && !SB16;  // the measurement variant's VALU dots
  u32x4 sn[2];  // BF16 pages: S_n of the even tile, stored with the odd one
  u32x4 sb[2];  // BF16 pages, align: S_me likewise
  char* const btile0 = static_cast<char*>(p.state) +
                       ((int64_t)bslot * p.slot_stride + (int64_t)h * PAGE +
                        (16 * (2 * wave) + lr) * K + LDC * lq) * ES;
  // The pass over the 16 tiles, compiled with and without the boundary stage
  // so that the common case carries no branch inside the unrolled loop.
  auto state_pass = [&](auto align_tag) {
    constexpr bool ALIGN = decltype(align_tag)::value;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int c0 = chan0<SB16>(cb, lq);
      const floatx4 xa = *reinterpret_cast<const floatx4*>(&x_s[lr][c0]);
      floatx4 dn4 = {1.f, 1.f, 1.f, 1.f};
      float ka0 = 0.f, ka1 = 0.f;
      // A operand row lr of the replay MFMA is the channel of accumulator row lr.
      const int ca = chan0<SB16>(cb, lr >> 2) + (lr & 3);
      if (replay) {
        dn4 = *reinterpret_cast<const floatx4*>(&dn_s[c0]);
        ka0 = kp_s[lq][ca];
        ka1 = kp_s[4 + lq][ca];
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        floatx4 s;
        if constexpr (SB16) {
          const u32x4 w = st[r][cb >> 1];
          const uint32_t w0 = (cb & 1) ? w[2] : w[0];
          const uint32_t w1 = (cb & 1) ? w[3] : w[1];
          s = floatx4{bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1)};
        } else {
          s = __builtin_bit_cast(floatx4, st[r][cb]);
        }
        if (replay) {
          const int64_t toff = (16 * r * K + 4 * LDC * (SB16 ? cb >> 1 : cb)) * ES;
          if constexpr (ALIGN) {
            // Stage one: S_me, stored to the boundary page.
            const floatx4 dm4 = *reinterpret_cast<const floatx4*>(&dm_s[c0]);
            s = s * dm4;
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(kpm_s[lq][ca], ub[r][0], s, 0, 0, 0);
            if (me > 4)
              s = __builtin_amdgcn_mfma_f32_16x16x4f32(kpm_s[4 + lq][ca], ub[r][1], s, 0, 0, 0);
            if constexpr (SB16) {
              sb[r][(cb & 1) * 2] = pack_bf16x2(s[0], s[1]);
              sb[r][(cb & 1) * 2 + 1] = pack_bf16x2(s[2], s[3]);
              if (cb & 1) *reinterpret_cast<u32x4*>(btile0 + toff) = sb[r];
            } else {
              *reinterpret_cast<floatx4*>(btile0 + toff) = s;
            }
          }
          s = s * dn4;
          s = __builtin_amdgcn_mfma_f32_16x16x4f32(ka0, ub[r][0], s, 0, 0, 0);
          if (n > 4) s = __builtin_amdgcn_mfma_f32_16x16x4f32(ka1, ub[r][1], s, 0, 0, 0);
          // S_n replaces the loaded page in the same registers; it is stored
          // at the end of the kernel.
          if constexpr (SB16) {
            sn[r][(cb & 1) * 2] = pack_bf16x2(s[0], s[1]);
            sn[r][(cb & 1) * 2 + 1] = pack_bf16x2(s[2], s[3]);
            if (cb & 1) st[r][cb >> 1] = sn[r];
          } else {
            st[r][cb] = __builtin_bit_cast(u32x4, s);
          }
        }
        if constexpr (!kValu) {
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[0], s[0], acc[r], 0, 0, 0);
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[1], s[1], acc[r], 0, 0, 0);
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[2], s[2], acc[r], 0, 0, 0);
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[3], s[3], acc[r], 0, 0, 0);
        }
      }
    }
  };
  if constexpr (FUSED) {
    if (balign)
      state_pass(std::true_type{});
    else
      state_pass(std::false_type{});
  } else {
    state_pass(std::false_type{});
  }
  // acc[r], lane l, value i: column j = 4(l/16) + i of state row 16(2w+r) + l%16.
  if constexpr (kShareXD) __syncthreads();  // every wave has read x_s: it now holds the dots
  if constexpr (kValu) {
    // The VALU variant's dots from S_n in the page registers (FP32 pages).
#pragma unroll 1
    for (int j = 0; j < 2 * T; ++j) {
      float a[2] = {0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const floatx4 x4 = *reinterpret_cast<const floatx4*>(&x_s[j][chan0<SB16>(cb, lq)]);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const floatx4 sv = __builtin_bit_cast(floatx4, st[r][cb]);
#pragma unroll
          for (int i = 0; i < 4; ++i) a[r] = fmaf(x4[i], sv[i], a[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        a[r] += __shfl_xor(a[r], 16);
        a[r] += __shfl_xor(a[r], 32);
        if (lq == 0) dots_s[j][16 * (2 * wave + r) + lr] = a[r];
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) dots_s[4 * lq + i][16 * (2 * wave + r) + lr] = acc[r][i];
  }
  __syncthreads();

  // ---- 6. Per state row: the T x T forward substitution, outputs, records.
  // The gated output stage keeps the BF16-rounded o in kp_s, whose last reads
  // were in the state pass.
  float (*const ob_s)[V] = reinterpret_cast<float (*)[V]>(&kp_s[0][0]);
  static_assert(MAX_T * K >= T * V, "o of the window fits in kp_s");
  if (lower) {
    const int vrow = c;
    float us[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float a = v_s[t][vrow] - dots_s[t][vrow];
#pragma unroll
      for (int s = 0; s < t; ++s) {
        const int ia = PI::a(t, s);
        a = fmaf(-pair_s[ia], us[s], a);
      }
      us[t] = beta_s[t] * a;
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float o = dots_s[T + t][vrow];
#pragma unroll
      for (int s = 0; s <= t; ++s) {
        const int ib = PI::b(t, s);
        o = fmaf(pair_s[ib], us[s], o);
      }
      if constexpr (GATED) {
        // The output stage normalises the BF16-rounded o over the head's rows.
        ob_s[t][vrow] = bf16_bits_to_f32(f32_to_bf16_bits(o));
      } else {
        if (t < L) {
          if constexpr (kWriteThrough) {
            // Write-through like the pages; the descriptor spans the item's
            // T token rows of this head.
            const __amdgpu_buffer_rsrc_t out_rs =
                page_rsrc(p.out + tok0 * H * V + (int64_t)h * V, (uint32_t)(T * H * V * 2));
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(o), out_rs,
                                                  (t * H * V + vrow) * 2, 0, CPOL_NT | CPOL_SC1);
          } else {
            p.out[(tok0 + t) * H * V + head_row] = f32_to_bf16_bits(o);
          }
        }
      }
    }
    if (rec >= 0) {
      const int64_t rbase = ((int64_t)rec * H + h) * p.rq;
      if constexpr (kWriteThrough) {
        // Write-through like the pages, within the item's record block.
        constexpr int CP = CPOL_NT | CPOL_SC1;
        const __amdgpu_buffer_rsrc_t corr_rs = page_rsrc(p.corr + rbase * V, p.rq * V * 4);
        const __amdgpu_buffer_rsrc_t kg_rs = page_rsrc(p.kg + rbase * 2 * K, p.rq * 2 * K * 2);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          if (t >= L) break;  // uniform
          const uint32_t bits = kg_s[t][c];
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(us[t]), corr_rs,
                                                (t * V + vrow) * 4, 0, CP);
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(bits & 0xffffu), kg_rs,
                                                (t * 2 * K + c) * 2, 0, CP);
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(bits >> 16), kg_rs,
                                                (t * 2 * K + K + c) * 2, 0, CP);
        }
      } else {
#pragma unroll
        for (int t = 0; t < T; ++t) {
          if (t >= L) break;  // uniform
          p.corr[(rbase + t) * V + vrow] = us[t];
          const uint32_t bits = kg_s[t][c];
          p.kg[(rbase + t) * 2 * K + c] = (uint16_t)(bits & 0xffffu);
          p.kg[(rbase + t) * 2 * K + K + c] = (uint16_t)(bits >> 16);
        }
      }
    }
  }
  if constexpr (GATED) {
    // All four waves finish the output: wave w tokens 2w and 2w + 1, the
    // sums of squares over the 128 rows by one wave reduction each.
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = 2 * wave + j;  // uniform
      if (t < L) {
        const float x0 = ob_s[t][lane], x1 = ob_s[t][lane + 64];
        const float ss = wave_sum(x0 * x0 + x1 * x1);
        const float rstd = __builtin_amdgcn_rsqf(ss * (1.0f / V) + p.norm_eps);
        uint16_t* const dst = p.out + (tok0 + t) * H * V + (int64_t)h * V;
        dst[lane] = (uint16_t)f32_to_bf16_bits(x0 * rstd * nw[0] *
                                               sigmoidf_fast(bf16_bits_to_f32(gtb[j][0])));
        dst[lane + 64] = (uint16_t)f32_to_bf16_bits(x1 * rstd * nw[1] *
                                                    sigmoidf_fast(bf16_bits_to_f32(gtb[j][1])));
      }
    }
  }
  // ---- 7. S_n back to the slot's page, last. Nothing in the kernel waits
  // for these stores, so with STREAM they write through the L2 (sc1) with the
  // no-reuse hint (nt) and leave no dirty lines behind.
  if constexpr (FUSED) {
    if (replay) {
      constexpr int CPOL = kWriteThrough ? (CPOL_NT | CPOL_SC1) : 0;
      const __amdgpu_buffer_rsrc_t page_rs = page_rsrc(page, PAGE * ES);
      const uint32_t tile_off = (uint32_t)(tile0 - page);
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int j = 0; j < NLD; ++j)
          store_page16<CPOL>(st[r][j], page_rs, tile_off + (16 * r * K + 4 * LDC * j) * ES);
    }
  }
}

// Launch of one fused instance: the streaming one when the grid's pages (batch
// x heads pages of 64 or 32 KiB) exceed the MALL. It writes through: on the
// 2 GiB FP32 pool of the large decode batch the step is 2.4% faster (the
// commit after it finds no dirty lines to write back), while pages that fit
// in the MALL are best kept there. Over FP32 pages it runs at two workgroups
// per CU; over BF16 pages at its natural four (two per CU made the step 9%
// slower), where the write-through stores took the 1 GiB pool's step from
// 0.879-0.885 to 0.858-0.861 ms (the fused launch 0.510-0.515 -> 0.497-0.500
// ms, the commit after it 0.358-0.362 -> 0.352-0.353 ms).
template <int TT, bool G, bool B, int MODE>
hipError_t launch_fused_instance(const VerifyParams& p, dim3 grid, hipStream_t stream) {
  if (stream_pages((int64_t)grid.x * grid.y * PAGE * (B ? 2 : 4))) {
    static const size_t pad =
        B ? 0 : two_per_cu_lds(&verify_kernel<TT, true, G, B, MODE, true>);
    hipLaunchKernelGGL((verify_kernel<TT, true, G, B, MODE, true>), grid, dim3(256), pad, stream,
                       p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((verify_kernel<TT, true, G, B, MODE, false>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

// Launch of the fused replay+verify with the convolution prologue over window
// layout MODE, for T = tokens, FP32 or BF16 pages, with or without the gated
// output stage.
template <int MODE>
hipError_t launch_conv_mode(const VerifyParams& p, int tokens, bool bf16, int batch,
                            hipStream_t stream) {
  const dim3 grid(p.heads, batch);
  const bool gated = p.gate != nullptr;
  hipError_t err = hipSuccess;
  auto launch = [&](auto t_tag, auto gated_tag, auto bf16_tag) {
    constexpr int TT = decltype(t_tag)::value;
    constexpr bool G = decltype(gated_tag)::value;
    constexpr bool B = decltype(bf16_tag)::value;
    err = launch_fused_instance<TT, G, B, MODE>(p, grid, stream);
  };
  auto by_page = [&](auto t_tag) {
    if (gated) {
      if (bf16) launch(t_tag, std::true_type{}, std::true_type{});
      else launch(t_tag, std::true_type{}, std::false_type{});
    } else {
      if (bf16) launch(t_tag, std::false_type{}, std::true_type{});
      else launch(t_tag, std::false_type{}, std::false_type{});
    }
  };
  switch (tokens) {
    case 1: by_page(std::integral_constant<int, 1>{}); break;
    case 2: by_page(std::integral_constant<int, 2>{}); break;
    case 3: by_page(std::integral_constant<int, 3>{}); break;
    case 4: by_page(std::integral_constant<int, 4>{}); break;
    case 5: by_page(std::integral_constant<int, 5>{}); break;
    case 6: by_page(std::integral_constant<int, 6>{}); break;
    case 7: by_page(std::integral_constant<int, 7>{}); break;
    case 8: by_page(std::integral_constant<int, 8>{}); break;
    default: return hipErrorInvalidValue;
  }
  return err;
}

}  // namespace kda
