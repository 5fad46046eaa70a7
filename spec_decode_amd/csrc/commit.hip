// RecoverSSM commit: folds n recorded tokens into a state page in closed form,
//   S_n = S_0 diag(D_n) + sum_{t<n} u_t (kn_t * P_t)^T,
// D_n = prod_{s<n} d_s and P_t = prod_{t<s<n} d_s, and with align also S_m to a
// boundary page (the vLLM page "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.
// commit": module docstring, KdaCommit class docstring and kernel).
//
// One workgroup of 256 threads (4 wave64) per (head, request, layer) item, in
// two kernels that share the item, the admission rules and the coefficients:
//
// - commit_kernel (BF16 pages, and FP32 pools that fit in the MALL): the page
//   goes HBM -> VGPRs -> HBM; each thread issues all of its 16-byte loads
//   before the coefficients are built and owns a fixed 16-byte column group
//   of every pass' rows, folded on the vector ALU. The LDS path below, run on
//   BF16 pages (32 KiB area, the same tiles in the fused kernel's BF16
//   channel order), lost: 8-layer align commit 1.13 against 0.974 ms, the
//   1 GiB pool's flush 0.398 against 0.355 ms; a BF16 page carries half the
//   bytes, so the path's per-item latency weighs twice as much.
// - commit_f32_stream_kernel (FP32 pages of launches larger than the MALL):
//   each wave loads its 32 rows as contiguous 1 KiB pieces, the first half
//   straight into its LDS area and the second half into registers, turns
//   both into 16x16 tiles in the accumulator layout of V_MFMA_F32_16X16X4_F32
//   through that area (as the stock verify loads its page), folds each tile
//   on the matrix cores (S^T <- diag(D) S^T + KP U^T, K = the replayed tokens)
//   and stores the tiles 16 rows per instruction, the access order that moves
//   the most on an in-place pass over a pool larger than the MALL.
//
// The two folds round in different orders (FP32 FMAs one token at a time,
// against the matrix cores' four-token sums), so an FP32 page committed by a
// launch above and by one below the MALL's size can differ in the last bits.
//
// Coefficients (thread c = key channel c of waves 0 and 1): decays of the
// recorded raw gates, the recorded raw keys normalised by their 128-channel
// L2 norm (eps 1e-6 inside the root), and suffix products walked from the
// last replayed token down: kp_t = kn_t * prod_{t<s<n} d_s, D_n. The commit
// page computes the same products in log space; the direct product is exact
// to FP32 rounding and needs no log or exp per token. With align, S_m is
// folded first, stored to the boundary page, and folded on to S_n (the commit
// composes: S_n is the commit of tokens m..n-1 onto S_m).
//
// STREAM (launches whose source pages exceed the 256 MB MALL) selects
// no-reuse page loads (nt) and write-through no-reuse page stores (sc1 nt) at
// two workgroups per CU: on the 2 GiB FP32 pool folded in place the launch is
// 9% faster with them, and so is the next launch on the pool (it finds no
// dirty lines of this one to write back), while launches whose pages fit in
// the MALL are about 5% slower with them.
#include "kda_device.h"

// A measurement variant, never built by default: with -DKDA_VALU_FOLD=1 the
// streaming FP32 commit folds its tiles with plain FP32 FMAs, one token at a
// time in the order of commit_kernel's fold (so its pages equal that kernel's
// bit for bit), instead of on the matrix cores. It exists to time the MFMA
// choice for this fold against the vector ALU on the same kernel.
#ifndef KDA_VALU_FOLD
#define KDA_VALU_FOLD 0
#endif

namespace kda {

constexpr bool kValuFold = KDA_VALU_FOLD != 0;

// Item of a workgroup and its admission (both kernels).
struct CommitItem {
  int h, b, n, ne, src, dst, row, mm, bnd;
};

// Returns false when the item commits nothing: no tokens, a null source or
// destination, or no record row. mm = the boundary length when a live
// boundary is given (capped at the tokens folded), else 0.
template <int Q, bool ALIGN>
__device__ __forceinline__ bool commit_item(const CommitParams& p, int h, int b, CommitItem& it) {
  it.h = h;
  it.b = b;
  it.n = p.lens[b];
  it.src = p.sources[b];
  it.dst = p.dests[b];
  it.row = p.rows != nullptr ? p.rows[b] : b;
  if (!(it.n > 0 && it.src > p.null_slot && it.dst > p.null_slot && it.row >= 0)) return false;
  it.ne = it.n < Q ? it.n : Q;
  it.mm = 0;
  it.bnd = p.null_slot;
  if constexpr (ALIGN) {
    const int m = p.blens[b];
    it.bnd = p.bounds[b];
    if (m > 0 && it.bnd > p.null_slot) it.mm = m < it.ne ? m : it.ne;
  }
  return true;
}

// Stage two's suffix products kp_t (tokens mm..ne-1 folded onto S_m; written
// for every t < ne) and D = prod_{mm<=s<ne} d_s, then with align stage one's
// kpm_t (t < mm) and D_m = prod_{s<mm} d_s. Thread c of the lower waves.
template <int Q, bool ALIGN>
__device__ __forceinline__ void commit_suffix_products(const float (&kn)[Q], const float (&d)[Q],
                                                       int ne, int mm, int c, float (*kp_s)[K],
                                                       float* dn_s, float (*kpm_s)[K],
                                                       float* dm_s) {
  float pp = 1.f, dmn = 1.f;
#pragma unroll
  for (int t = Q - 1; t >= 0; --t) {
    if (t < ne) {
      kp_s[t][c] = kn[t] * pp;
      pp *= d[t];
      if (t == mm) dmn = pp;
    }
  }
  dn_s[c] = dmn;
  if constexpr (ALIGN) {
    if (mm > 0) {
      float pm = 1.f;
#pragma unroll
      for (int t = Q - 1; t >= 0; --t) {
        if (t < mm) {
          kpm_s[t][c] = kn[t] * pm;
          pm *= d[t];
        }
      }
      dm_s[c] = pm;
    }
  }
}

// ------------------------------------------------------------ FP32 pages

// One stage of the fold over tokens t0 <= t < t1 on the tiles:
// S^T <- diag(D) S^T + KP U^T. In V_MFMA_F32_16X16X4_F32 terms the tile is the
// accumulator (M = key channel, N = state row), A = kp_t[c] (lane l: channel
// 16cb + l%16, token l/16 of the MFMA's four) and B = u_t[v] (lane l: token
// l/16, row l%16). ub[r][j] holds u of token 4j + l/16 at the lane's row of
// tile row r, zero past the last folded token; tokens outside the stage get
// a zero A operand.
template <int Q>
__device__ __forceinline__ void fold_tiles(u32x4 (&st)[2][8], const float (&ub)[2][2],
                                           const float* D, const float (*kp)[K], int t0, int t1,
                                           int lane) {
  const int lr = lane & 15, lq = lane >> 4;
  const bool mf0 = t0 < (t1 < 4 ? t1 : 4);  // wave-uniform: a token of 0..3 in the stage
  const bool mf1 = t1 > (t0 > 4 ? t0 : 4);  // and of 4..7
  const bool in0 = lq >= t0 && lq < t1;
  const bool in1 = 4 + lq >= t0 && 4 + lq < t1;
  const int k0 = lq < Q ? lq : Q - 1;
  const int k1 = 4 + lq < Q ? 4 + lq : Q - 1;
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    const floatx4 dd = *reinterpret_cast<const floatx4*>(D + 16 * cb + 4 * lq);
    const float ka0 = in0 ? kp[k0][16 * cb + lr] : 0.f;
    const float ka1 = in1 ? kp[k1][16 * cb + lr] : 0.f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      floatx4 s = __builtin_bit_cast(floatx4, st[r][cb]) * dd;
      if (mf0) s = __builtin_amdgcn_mfma_f32_16x16x4f32(ka0, ub[r][0], s, 0, 0, 0);
      if (mf1) s = __builtin_amdgcn_mfma_f32_16x16x4f32(ka1, ub[r][1], s, 0, 0, 0);
      st[r][cb] = __builtin_bit_cast(u32x4, s);
    }
  }
}

// The measurement variant's fold of the same tiles on the vector ALU:
// s <- s D + sum_{t0 <= t < t1} u_t kp_t element by element, one FMA per
// token. uu[r][t] holds u_t at the lane's row of tile row r (zero past the
// last folded token); the lane's 4 channels of tile cb are 16cb + 4(l/16)...
template <int Q>
__device__ __forceinline__ void fold_tiles_valu(u32x4 (&st)[2][8], const float (&uu)[2][Q],
                                                const float* D, const float (*kp)[K], int t0,
                                                int t1, int lane) {
  const int c4 = 4 * (lane >> 4);
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    const floatx4 dd = *reinterpret_cast<const floatx4*>(D + 16 * cb + c4);
    floatx4 s0 = __builtin_bit_cast(floatx4, st[0][cb]) * dd;
    floatx4 s1 = __builtin_bit_cast(floatx4, st[1][cb]) * dd;
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      if (t >= t0 && t < t1) {
        const floatx4 k = *reinterpret_cast<const floatx4*>(&kp[t][16 * cb + c4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s0[e] = fmaf(uu[0][t], k[e], s0[e]);
          s1[e] = fmaf(uu[1][t], k[e], s1[e]);
        }
      }
    }
    st[0][cb] = __builtin_bit_cast(u32x4, s0);
    st[1][cb] = __builtin_bit_cast(u32x4, s1);
  }
}

// The tiles back to a page, consecutive rows with the column blocks inner.
template <int CPOL>
__device__ __forceinline__ void store_tiles(const u32x4 (&st)[2][8], float* page, int wave,
                                            int lane) {
  const __amdgpu_buffer_rsrc_t rs = page_rsrc(page, PAGE * 4);
  const uint32_t off0 = (uint32_t)(((32 * wave + (lane & 15)) * K + 4 * (lane >> 4)) * 4);
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      store_page16<CPOL>(st[r][cb], rs, off0 + (16 * r * K + 16 * cb) * 4);
}

// FP32 pages of launches larger than the MALL, at two workgroups per CU (the
// occupancy its write-through stores want; its 41 KiB of LDS would allow
// three, which was slower). The key norms are formed within each of waves 0
// and 1 (each lane also loads the channel of the other wave), so the kernel's
// one barrier is the one before the fold, which waits for the page, needed
// next anyway. On the large decode flush (2 GiB pool, in place) it takes
// 0.622-0.624 ms, against 0.629-0.633 ms with the whole page straight into a
// 64 KiB LDS area, 0.644 ms with the tiles folded on the vector ALU, and
// 0.650-0.652 ms for commit_kernel. For pools that fit in the MALL
// commit_kernel is the faster one (24.6 against 28.8 us on 68 MiB, 64 against
// 69 us on 196 MiB, measured with the 64 KiB area): at its four workgroups per
// CU latency hides better, and the LDS area or tile-order register loads
// (28.0 and 69 us) cost more than they save there.
template <int Q, bool ALIGN>
__global__ __launch_bounds__(256) void commit_f32_stream_kernel(const CommitParams p) {
  CommitItem it;
  if (!commit_item<Q, ALIGN>(p, blockIdx.x, blockIdx.y, it)) return;
  const int l = blockIdx.z;
  const int tid = threadIdx.x;
  const CommitLayer L = p.layer[l];
  const int H = p.heads;

  __shared__ __attribute__((aligned(16))) u32x4 xt_s[4][16 * 32];  // per-wave transpose areas
  __shared__ float u_s[Q][V];
  __shared__ __attribute__((aligned(16))) float kp_s[Q][K];
  __shared__ __attribute__((aligned(16))) float dn_s[K];
  __shared__ float kpm_s[ALIGN ? Q : 1][K];
  __shared__ __attribute__((aligned(16))) float dm_s[ALIGN ? K : 1];

  const int lane = tid & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const bool lower = wave < 2;  // waves 0, 1: key channels; 2, 3: corrections
  const int c = tid & (K - 1);
  const int ne = it.ne, mm = it.mm;
  uint32_t kb[Q], ko[Q], gb[Q];
  float uval[Q];
  const float a_log_lh = p.a_log[l * H + it.h];
  const float dtb = p.dt_bias[((int64_t)l * H + it.h) * K + c];
  {
    // Branch-free record loads (token index clamped, values masked later):
    // the channel's key, gate and correction, and the key of channel c ^ 64
    // for the norm. They go first: loads return in order, so the
    // coefficients can start while the page is still streaming in.
    const int64_t tok0 = (int64_t)it.h * Q;
    const uint16_t* kg = L.kg + (int64_t)it.row * L.kg_stride + tok0 * 2 * K;
    const float* corr = L.corr + (int64_t)it.row * L.corr_stride + tok0 * V;
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      const int tt = t < ne ? t : 0;
      kb[t] = kg[tt * 2 * K + c];
      ko[t] = kg[tt * 2 * K + (c ^ 64)];
      gb[t] = kg[tt * 2 * K + K + c];
      uval[t] = corr[tt * V + c];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const float* srcp = reinterpret_cast<const float*>(L.state) + (int64_t)it.src * L.state_stride +
                      (int64_t)it.h * PAGE;
  u32x4 cont[8];
  load_page_halves(srcp, wave, lane, &xt_s[wave][0], cont);
  __builtin_amdgcn_sched_barrier(0);

  if (lower) {
    const float ea = __expf(a_log_lh);
    float d[Q], kn[Q];
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      d[t] = 1.f;
      kn[t] = 0.f;
      if (t < ne) {
        const float kraw = bf16_bits_to_f32(kb[t]);
        const float koth = bf16_bits_to_f32(ko[t]);
        d[t] = gate_decay(bf16_bits_to_f32(gb[t]), ea, dtb, p.lb);
        const float ss = wave_sum(kraw * kraw) + wave_sum(koth * koth);
        kn[t] = kraw * __builtin_amdgcn_rsqf(ss + 1e-6f);
      }
    }
    commit_suffix_products<Q, ALIGN>(kn, d, ne, mm, c, kp_s, dn_s, kpm_s, dm_s);
  } else {
#pragma unroll
    for (int t = 0; t < Q; ++t)
      if (t < ne) u_s[t][c] = uval[t];
  }
  __syncthreads();

  u32x4 st[2][8];
  transpose_page_halves(cont, &xt_s[wave][0], lane, st);
  float ub[2][2];
  {
    const int lq = lane >> 4;
    const int k0 = lq < Q ? lq : Q - 1;
    const int k1 = 4 + lq < Q ? 4 + lq : Q - 1;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int vrow = 32 * wave + 16 * r + (lane & 15);
      ub[r][0] = lq < ne ? u_s[k0][vrow] : 0.f;
      ub[r][1] = 4 + lq < ne ? u_s[k1][vrow] : 0.f;
    }
  }
  float uu[kValuFold ? 2 : 1][kValuFold ? Q : 1];
  if constexpr (kValuFold) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int t = 0; t < Q; ++t)
        uu[r][t] = t < ne ? u_s[t][32 * wave + 16 * r + (lane & 15)] : 0.f;
  }
  auto fold = [&](const float* D, const float (*kp)[K], int t0, int t1) {
    if constexpr (kValuFold)
      fold_tiles_valu<Q>(st, uu, D, kp, t0, t1, lane);
    else
      fold_tiles<Q>(st, ub, D, kp, t0, t1, lane);
  };
  float* base = reinterpret_cast<float*>(L.state);
  if constexpr (ALIGN) {
    if (mm > 0) {
      fold(&dm_s[0], kpm_s, 0, mm);
      store_tiles<CPOL_NT | CPOL_SC1>(
          st, base + (int64_t)it.bnd * L.state_stride + (int64_t)it.h * PAGE, wave, lane);
    }
  }
  fold(&dn_s[0], kp_s, mm, ne);
  store_tiles<CPOL_NT | CPOL_SC1>(
      st, base + (int64_t)it.dst * L.state_stride + (int64_t)it.h * PAGE, wave, lane);
}

// ------------------------------------------------------------ register path

// s[i][e] <- s[i][e] * D[c0 + e] + sum_{t0 <= t < t1} u[t][r0 + RPP i] * kp[t][c0 + e]
template <int EPC, int PASSES, int RPP, int Q>
__device__ __forceinline__ void fold_stage(float (&s)[PASSES][EPC], const float* D,
                                           const float* kp, const float* u, int t0, int t1,
                                           int c0, int r0) {
  float dd[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) dd[e] = D[c0 + e];
#pragma unroll
  for (int i = 0; i < PASSES; ++i)
#pragma unroll
    for (int e = 0; e < EPC; ++e) s[i][e] *= dd[e];
#pragma unroll
  for (int t = 0; t < Q; ++t) {
    if (t >= t0 && t < t1) {
      float k[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) k[e] = kp[t * K + c0 + e];
#pragma unroll
      for (int i = 0; i < PASSES; ++i) {
        const float uu = u[t * V + r0 + RPP * i];
#pragma unroll
        for (int e = 0; e < EPC; ++e) s[i][e] = fmaf(uu, k[e], s[i][e]);
      }
    }
  }
}

// The page's 16-byte chunks, rounded to the state dtype (BF16: nearest-even).
template <bool BF16, bool STREAM, int EPC, int PASSES, int RPP, typename Elem>
__device__ __forceinline__ void store_page(const float (&s)[PASSES][EPC], Elem* pg, int c0,
                                           int r0) {
  const __amdgpu_buffer_rsrc_t rs = page_rsrc(pg, PAGE * (int)sizeof(Elem));
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    u32x4 w;
    if constexpr (BF16) {
      w[0] = pack_bf16x2(s[i][0], s[i][1]);
      w[1] = pack_bf16x2(s[i][2], s[i][3]);
      w[2] = pack_bf16x2(s[i][4], s[i][5]);
      w[3] = pack_bf16x2(s[i][6], s[i][7]);
    } else {
      w[0] = __float_as_uint(s[i][0]);
      w[1] = __float_as_uint(s[i][1]);
      w[2] = __float_as_uint(s[i][2]);
      w[3] = __float_as_uint(s[i][3]);
    }
    const uint32_t off = (uint32_t)(((r0 + RPP * i) * K + c0) * (int)sizeof(Elem));
    store_page16<STREAM ? (CPOL_NT | CPOL_SC1) : 0>(w, rs, off);
  }
}

template <bool BF16, int Q, bool ALIGN, bool STREAM>
__global__ __launch_bounds__(256) void commit_kernel(const CommitParams p) {
  using Elem = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int EPC = 16 / (int)sizeof(Elem);  // elements per 16-byte chunk
  constexpr int CPR = K / EPC;                 // chunks per state row
  constexpr int RPP = 256 / CPR;               // rows per pass of the workgroup
  constexpr int PASSES = V / RPP;

  // Item order. Workgroups are dealt to the 8 XCDs round-robin by linear
  // index; the streaming align instances remap that index so that XCD x
  // takes the x-th eighth of the layer's (head, request) items, i.e. whole
  // requests' pages in turn, instead of every eighth head of the requests in
  // flight: the 8-layer BF16 align commit 1.050 -> 0.975 ms (1.045 against
  // 0.975 ms when re-measured). Commits without boundaries keep the launch
  // order, as the fused step does: the 1 GiB BF16 in-place flush after the
  // fused step took 0.351-0.352 ms with the remap against 0.337-0.339 ms
  // without. Unsigned: heads x batch reaches 65535^2, above INT_MAX but below
  // 2^32.
  uint32_t lin = blockIdx.x + blockIdx.y * gridDim.x;
  if constexpr (STREAM && ALIGN) {
    const uint32_t per_layer = gridDim.x * gridDim.y;
    if ((per_layer & 7u) == 0) lin = (lin & 7u) * (per_layer >> 3) + (lin >> 3);
  }
  CommitItem it;
  if (!commit_item<Q, ALIGN>(p, (int)(lin % gridDim.x), (int)(lin / gridDim.x), it)) return;
  const int l = blockIdx.z;
  const int tid = threadIdx.x;
  const CommitLayer L = p.layer[l];
  const int H = p.heads;

  __shared__ float u_s[Q][V];
  __shared__ float kp_s[Q][K];
  __shared__ float dn_s[K];
  __shared__ float kpm_s[ALIGN ? Q : 1][K];
  __shared__ float dm_s[ALIGN ? K : 1];
  __shared__ float ssq_s[2][Q];

  // ---- 1-2. Loads. The record loads go first, branch-free (token index
  // clamped, values masked later) and kept raw, then the page loads right
  // behind them: loads return in order, so the coefficient work below can start
  // when the records arrive while the page is still streaming in.
  const int lane = tid & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const bool lower = wave < 2;  // waves 0, 1: key channels; 2, 3: corrections
  const int c = tid & (K - 1);
  const int ne = it.ne, mm = it.mm;
  uint32_t kb[Q], gb[Q];
  float uval[Q];
  const int c0 = (tid % CPR) * EPC;
  const int r0 = tid / CPR;
  const Elem* srcp = reinterpret_cast<const Elem*>(L.state) + (int64_t)it.src * L.state_stride +
                     (int64_t)it.h * PAGE;
  uint4 raw[PASSES];
  const float a_log_lh = p.a_log[l * H + it.h];
  const float dtb = p.dt_bias[((int64_t)l * H + it.h) * K + c];
  {
    // Branch-free: every thread loads its channel's recorded key, gate and
    // correction (each half of the workgroup uses one of them; the duplicate
    // reads hit L2), so no value is defined on one path only.
    const int64_t tok0 = (int64_t)it.h * Q;
    const uint16_t* kg = L.kg + (int64_t)it.row * L.kg_stride + tok0 * 2 * K;
    const float* corr = L.corr + (int64_t)it.row * L.corr_stride + tok0 * V;
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      const int tt = t < ne ? t : 0;
      kb[t] = kg[tt * 2 * K + c];
      gb[t] = kg[tt * 2 * K + K + c];
      uval[t] = corr[tt * V + c];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const u32x4* const ptr = reinterpret_cast<const u32x4*>(srcp + (r0 + RPP * i) * K + c0);
    const u32x4 w = STREAM ? __builtin_nontemporal_load(ptr) : *ptr;
    raw[i] = uint4{w[0], w[1], w[2], w[3]};
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. Per-channel coefficients.
  float d[Q], kraw[Q];
  if (lower) {
    const float ea = __expf(a_log_lh);
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      d[t] = 1.f;
      kraw[t] = 0.f;
      if (t < ne) {
        kraw[t] = bf16_bits_to_f32(kb[t]);
        d[t] = gate_decay(bf16_bits_to_f32(gb[t]), ea, dtb, p.lb);
        const float s = wave_sum(kraw[t] * kraw[t]);
        if (lane == 0) ssq_s[wave][t] = s;
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < Q; ++t)
      if (t < ne) u_s[t][c] = uval[t];
  }
  __syncthreads();
  if (lower) {
    float kn[Q];
#pragma unroll
    for (int t = 0; t < Q; ++t)
      kn[t] = t < ne ? kraw[t] * __builtin_amdgcn_rsqf(ssq_s[0][t] + ssq_s[1][t] + 1e-6f) : 0.f;
    commit_suffix_products<Q, ALIGN>(kn, d, ne, mm, c, kp_s, dn_s, kpm_s, dm_s);
  }
  __syncthreads();

  // ---- 4. The fold, in registers: per stage s = s diag(D) + sum_t u_t kp_t.
  float s[PASSES][EPC];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    if constexpr (BF16) {
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[i][2 * j] = bf16_lo(w[j]);
        s[i][2 * j + 1] = bf16_hi(w[j]);
      }
    } else {
      s[i][0] = __uint_as_float(raw[i].x);
      s[i][1] = __uint_as_float(raw[i].y);
      s[i][2] = __uint_as_float(raw[i].z);
      s[i][3] = __uint_as_float(raw[i].w);
    }
  }
  Elem* base = reinterpret_cast<Elem*>(L.state);
  if constexpr (ALIGN) {
    if (mm > 0) {
      fold_stage<EPC, PASSES, RPP, Q>(s, &dm_s[0], &kpm_s[0][0], &u_s[0][0], 0, mm, c0, r0);
      store_page<BF16, STREAM, EPC, PASSES, RPP>(
          s, base + (int64_t)it.bnd * L.state_stride + (int64_t)it.h * PAGE, c0, r0);
    }
  }
  fold_stage<EPC, PASSES, RPP, Q>(s, &dn_s[0], &kp_s[0][0], &u_s[0][0], mm, ne, c0, r0);
  store_page<BF16, STREAM, EPC, PASSES, RPP>(
      s, base + (int64_t)it.dst * L.state_stride + (int64_t)it.h * PAGE, c0, r0);
}

// ------------------------------------------------------------ launch

template <bool BF16, bool ALIGN, bool STREAM>
static hipError_t launch_q(const CommitParams& p, int window, dim3 grid, hipStream_t stream) {
  switch (window) {
#define KDA_COMMIT_CASE(QQ)                                                                   \
  case QQ: {                                                                                 \
    if constexpr (STREAM && !BF16) {                                                         \
      static const size_t pad = two_per_cu_lds(&commit_f32_stream_kernel<QQ, ALIGN>);       \
      hipLaunchKernelGGL((commit_f32_stream_kernel<QQ, ALIGN>), grid, dim3(256), pad, stream, \
                         p);                                                                 \
    } else {                                                                                 \
      static const size_t pad =                                                              \
          STREAM ? two_per_cu_lds(&commit_kernel<BF16, QQ, ALIGN, STREAM>) : 0;              \
      hipLaunchKernelGGL((commit_kernel<BF16, QQ, ALIGN, STREAM>), grid, dim3(256), pad,     \
                         stream, p);                                                         \
    }                                                                                        \
    break;                                                                                   \
  }
    KDA_COMMIT_CASE(1)
    KDA_COMMIT_CASE(2)
    KDA_COMMIT_CASE(3)
    KDA_COMMIT_CASE(4)
    KDA_COMMIT_CASE(5)
    KDA_COMMIT_CASE(6)
    KDA_COMMIT_CASE(7)
    KDA_COMMIT_CASE(8)
#undef KDA_COMMIT_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_commit(const CommitParams& p, int window, bool bf16, bool align, int batch,
                         int layers, hipStream_t stream) {
  const dim3 grid(p.heads, batch, layers);
  // The source pages the launch can read (every request taken as live).
  const bool st = stream_pages((int64_t)batch * p.heads * layers * PAGE * (bf16 ? 2 : 4));
  if (bf16) {
    if (align) return st ? launch_q<true, true, true>(p, window, grid, stream)
                         : launch_q<true, true, false>(p, window, grid, stream);
    return st ? launch_q<true, false, true>(p, window, grid, stream)
              : launch_q<true, false, false>(p, window, grid, stream);
  }
  if (align) return st ? launch_q<false, true, true>(p, window, grid, stream)
                       : launch_q<false, true, false>(p, window, grid, stream);
  return st ? launch_q<false, false, true>(p, window, grid, stream)
            : launch_q<false, false, false>(p, window, grid, stream);
}

}  // namespace kda
