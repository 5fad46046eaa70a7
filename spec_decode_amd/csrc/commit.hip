// RecoverSSM commit: folds n recorded tokens into a state page in closed form,
//   S_n = S_0 diag(D_n) + sum_{t<n} u_t (kn_t * P_t)^T,
// D_n = prod_{s<n} d_s and P_t = prod_{t<s<n} d_s, and with align also S_m to a
// boundary page (the vLLM page "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.
// commit": module docstring, KdaCommit class docstring and kernel).
//
// One workgroup of 256 threads (4 wave64) per (head, request, layer) item. The
// page goes HBM -> VGPRs -> HBM once: each thread issues all of its 16-byte
// loads (8 for a 32 KiB BF16 page, 16 for a 64 KiB FP32 page) before the
// per-channel coefficients are built, so the page streams in while the decays
// are computed; the registers are the staging buffer (no LDS round trip).
// Thread tid owns a fixed 16-byte column group of every pass' rows, so the
// coefficient vectors it needs are a few LDS reads per token.
//
// Coefficients (threads 0..127, thread c = key channel c): decays of the
// recorded raw gates, the recorded raw keys normalised by their 128-channel
// L2 norm (eps 1e-6 inside the root), and suffix products walked from the
// last replayed token down: kp_t = kn_t * prod_{t<s<n} d_s, D_n. The commit
// page computes the same products in log space; the direct product is exact
// to FP32 rounding and needs no log or exp per token. With align, S_m is
// folded first, stored to the boundary page, and folded on to S_n.
#include "kda_device.h"

namespace kda {

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
// STREAM: write-through no-reuse stores (see commit_kernel).
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

// STREAM selects no-reuse page loads (nt) and write-through no-reuse page
// stores (sc1 nt), launched at two workgroups per CU. They pay off only when
// a launch's pages exceed the 256 MB MALL: on the 2 GiB FP32 pool folded in
// place the launch is 9% faster, and so is the next launch on the pool (it
// finds no dirty lines of this one to write back), while launches whose pages
// fit in the MALL are about 5% slower with them. The launcher chooses by the
// page bytes the launch can read.
template <bool BF16, int Q, bool ALIGN, bool STREAM>
__global__ __launch_bounds__(256) void commit_kernel(const CommitParams p) {
  using Elem = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int EPC = 16 / (int)sizeof(Elem);  // elements per 16-byte chunk
  constexpr int CPR = K / EPC;                 // chunks per state row
  constexpr int RPP = 256 / CPR;               // rows per pass of the workgroup
  constexpr int PASSES = V / RPP;

  // Item order. Workgroups are dealt to the 8 XCDs round-robin by linear
  // index; the streaming instances remap that index so that XCD x takes the
  // x-th eighth of the layer's (head, request) items, i.e. whole requests'
  // pages in turn, instead of every eighth head of the requests in flight
  // (large decode FP32 commit 0.662 -> 0.650 ms, 8-layer align 1.050 ->
  // 0.975 ms; the 1 GiB BF16 in-place commit 0.347 -> 0.357 ms).
  // Unsigned: heads x batch reaches 65535^2, above INT_MAX but below 2^32.
  uint32_t lin = blockIdx.x + blockIdx.y * gridDim.x;
  if constexpr (STREAM) {
    const uint32_t per_layer = gridDim.x * gridDim.y;
    if ((per_layer & 7u) == 0) lin = (lin & 7u) * (per_layer >> 3) + (lin >> 3);
  }
  const int h = (int)(lin % gridDim.x);
  const int b = (int)(lin / gridDim.x);
  const int l = blockIdx.z;
  const int tid = threadIdx.x;

  const int n = p.lens[b];
  const int src = p.sources[b];
  const int dst = p.dests[b];
  const int row = p.rows != nullptr ? p.rows[b] : b;
  if (!(n > 0 && src > p.null_slot && dst > p.null_slot && row >= 0)) return;
  const int ne = n < Q ? n : Q;
  int me = 0;
  int bnd = p.null_slot;
  bool blive = false;
  if constexpr (ALIGN) {
    const int m = p.blens[b];
    bnd = p.bounds[b];
    blive = m > 0 && bnd > p.null_slot;
    me = m < ne ? m : ne;
  }
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
  const int64_t rec_tok0 = ((int64_t)h * Q);
  uint32_t kb[Q], gb[Q];
  float uval[Q];
  const int c0 = (tid % CPR) * EPC;
  const int r0 = tid / CPR;
  const Elem* srcp =
      reinterpret_cast<const Elem*>(L.state) + (int64_t)src * L.state_stride + (int64_t)h * PAGE;
  uint4 raw[PASSES];
  const float a_log_lh = p.a_log[l * H + h];
  const float dtb = p.dt_bias[((int64_t)l * H + h) * K + c];
  {
    // Branch-free: every thread loads its channel's recorded key, gate and
    // correction (each half of the workgroup uses one of them; the duplicate
    // reads hit L2), so no value is defined on one path only.
    const uint16_t* kg = L.kg + (int64_t)row * L.kg_stride + rec_tok0 * 2 * K;
    const float* corr = L.corr + (int64_t)row * L.corr_stride + rec_tok0 * V;
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
  for (int i = 0; i < PASSES; ++i)
  {
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
  // With a live boundary the fold runs in two stages through S_m (the commit
  // composes: S_n is the commit of tokens m..n-1 onto S_m), so one accumulator
  // serves both stores. mm = m when the boundary is live, else 0.
  const int mm = (ALIGN && blive) ? me : 0;
  if (lower) {
    float kn[Q];
#pragma unroll
    for (int t = 0; t < Q; ++t)
      kn[t] = t < ne ? kraw[t] * __builtin_amdgcn_rsqf(ssq_s[0][t] + ssq_s[1][t] + 1e-6f) : 0.f;
    // Stage two (tokens mm..ne-1): kp_t = kn_t prod_{t<s<ne} d_s, D = prod_{mm<=s<ne} d_s.
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
    // Stage one (tokens 0..mm-1): kpm_t = kn_t prod_{t<s<mm} d_s, D_m = prod_{s<mm} d_s.
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
      store_page<BF16, STREAM, EPC, PASSES, RPP>(s, base + (int64_t)bnd * L.state_stride + (int64_t)h * PAGE,
                                         c0, r0);
    }
  }
  fold_stage<EPC, PASSES, RPP, Q>(s, &dn_s[0], &kp_s[0][0], &u_s[0][0], mm, ne, c0, r0);
  store_page<BF16, STREAM, EPC, PASSES, RPP>(s, base + (int64_t)dst * L.state_stride + (int64_t)h * PAGE,
                                     c0, r0);
}

template <bool BF16, bool ALIGN, bool STREAM>
static hipError_t launch_q(const CommitParams& p, int window, dim3 grid, hipStream_t stream) {
  switch (window) {
#define KDA_COMMIT_CASE(QQ)                                                                 \
  case QQ: {                                                                               \
    static const size_t pad =                                                              \
        STREAM ? two_per_cu_lds(&commit_kernel<BF16, QQ, ALIGN, STREAM>) : 0;              \
    hipLaunchKernelGGL((commit_kernel<BF16, QQ, ALIGN, STREAM>), grid, dim3(256), pad,     \
                       stream, p);                                                         \
    break;                                                                                 \
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
