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
// to FP32 rounding and needs no log or exp per token.
#include "kda_device.h"

namespace kda {

template <bool BF16, int Q, bool ALIGN>
__global__ __launch_bounds__(256) void commit_kernel(const CommitParams p) {
  using Elem = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int EPC = 16 / (int)sizeof(Elem);  // elements per 16-byte chunk
  constexpr int CPR = K / EPC;                 // chunks per state row
  constexpr int RPP = 256 / CPR;               // rows per pass of the workgroup
  constexpr int PASSES = V / RPP;

  const int h = blockIdx.x;
  const int b = blockIdx.y;
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

  // ---- 1. Record loads (issued first so the page loads queue behind them).
  const int64_t rec_tok0 = ((int64_t)h * Q);
  float kraw[Q], graw[Q], uval[Q];
  if (tid < K) {
    const uint16_t* kg = L.kg + (int64_t)row * L.kg_stride + rec_tok0 * 2 * K;
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      kraw[t] = 0.f;
      graw[t] = 0.f;
      if (t < ne) {
        kraw[t] = bf16_bits_to_f32(kg[t * 2 * K + tid]);
        graw[t] = bf16_bits_to_f32(kg[t * 2 * K + K + tid]);
      }
    }
  } else {
    const float* corr = L.corr + (int64_t)row * L.corr_stride + rec_tok0 * V;
#pragma unroll
    for (int t = 0; t < Q; ++t) uval[t] = t < ne ? corr[t * V + (tid - K)] : 0.f;
  }

  // ---- 2. The source page: PASSES 16-byte chunks per thread, in flight.
  const int c0 = (tid % CPR) * EPC;
  const int r0 = tid / CPR;
  const Elem* srcp =
      reinterpret_cast<const Elem*>(L.state) + (int64_t)src * L.state_stride + (int64_t)h * PAGE;
  uint4 raw[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i)
    raw[i] = *reinterpret_cast<const uint4*>(srcp + (r0 + RPP * i) * K + c0);

  // ---- 3. Per-channel coefficients.
  const int lane = tid & (WAVE - 1);
  const int wave = tid / WAVE;
  float d[Q];
  if (tid < K) {
    const float ea = __expf(p.a_log[l * H + h]);
    const float dtb = p.dt_bias[((int64_t)l * H + h) * K + tid];
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      d[t] = 1.f;
      if (t < ne) {
        d[t] = gate_decay(graw[t], ea, dtb, p.lb);
        const float s = wave_sum(kraw[t] * kraw[t]);
        if (lane == 0) ssq_s[wave][t] = s;
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < Q; ++t)
      if (t < ne) u_s[t][tid - K] = uval[t];
  }
  __syncthreads();
  if (tid < K) {
    float kn[Q];
#pragma unroll
    for (int t = 0; t < Q; ++t)
      kn[t] = t < ne ? kraw[t] * __builtin_amdgcn_rsqf(ssq_s[0][t] + ssq_s[1][t] + 1e-6f) : 0.f;
    float pp = 1.f;
#pragma unroll
    for (int t = Q - 1; t >= 0; --t) {
      if (t < ne) {
        kp_s[t][tid] = kn[t] * pp;
        pp *= d[t];
      }
    }
    dn_s[tid] = pp;
    if constexpr (ALIGN) {
      if (blive) {
        float pm = 1.f;
#pragma unroll
        for (int t = Q - 1; t >= 0; --t) {
          if (t < me) {
            kpm_s[t][tid] = kn[t] * pm;
            pm *= d[t];
          }
        }
        dm_s[tid] = pm;
      }
    }
  }
  __syncthreads();

  // ---- 4. The fold, in registers: s = S_0 diag(D) then += u_t kp_t per token.
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
  float sb[ALIGN ? PASSES : 1][EPC];
  {
    float dn[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) dn[e] = dn_s[c0 + e];
    if constexpr (ALIGN) {
      if (blive) {
        float dm[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) dm[e] = dm_s[c0 + e];
#pragma unroll
        for (int i = 0; i < PASSES; ++i)
#pragma unroll
          for (int e = 0; e < EPC; ++e) sb[i][e] = s[i][e] * dm[e];
      }
    }
#pragma unroll
    for (int i = 0; i < PASSES; ++i)
#pragma unroll
      for (int e = 0; e < EPC; ++e) s[i][e] *= dn[e];
  }
#pragma unroll
  for (int t = 0; t < Q; ++t) {
    if (t < ne) {
      float kp[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) kp[e] = kp_s[t][c0 + e];
      const bool bt = ALIGN && blive && t < me;
      float kpm[EPC];
      if constexpr (ALIGN) {
        if (bt) {
#pragma unroll
          for (int e = 0; e < EPC; ++e) kpm[e] = kpm_s[t][c0 + e];
        }
      }
#pragma unroll
      for (int i = 0; i < PASSES; ++i) {
        const float u = u_s[t][r0 + RPP * i];
#pragma unroll
        for (int e = 0; e < EPC; ++e) s[i][e] = fmaf(u, kp[e], s[i][e]);
        if constexpr (ALIGN) {
          if (bt) {
#pragma unroll
            for (int e = 0; e < EPC; ++e) sb[i][e] = fmaf(u, kpm[e], sb[i][e]);
          }
        }
      }
    }
  }

  // ---- 5. Stores: destination (and boundary) page, 16 bytes per chunk.
  Elem* base = reinterpret_cast<Elem*>(L.state);
  Elem* dstp = base + (int64_t)dst * L.state_stride + (int64_t)h * PAGE;
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    uint4 w;
    if constexpr (BF16) {
      w.x = pack_bf16x2(s[i][0], s[i][1]);
      w.y = pack_bf16x2(s[i][2], s[i][3]);
      w.z = pack_bf16x2(s[i][4], s[i][5]);
      w.w = pack_bf16x2(s[i][6], s[i][7]);
    } else {
      w.x = __float_as_uint(s[i][0]);
      w.y = __float_as_uint(s[i][1]);
      w.z = __float_as_uint(s[i][2]);
      w.w = __float_as_uint(s[i][3]);
    }
    *reinterpret_cast<uint4*>(dstp + (r0 + RPP * i) * K + c0) = w;
  }
  if constexpr (ALIGN) {
    if (blive) {
      Elem* bp = base + (int64_t)bnd * L.state_stride + (int64_t)h * PAGE;
#pragma unroll
      for (int i = 0; i < PASSES; ++i) {
        uint4 w;
        if constexpr (BF16) {
          w.x = pack_bf16x2(sb[i][0], sb[i][1]);
          w.y = pack_bf16x2(sb[i][2], sb[i][3]);
          w.z = pack_bf16x2(sb[i][4], sb[i][5]);
          w.w = pack_bf16x2(sb[i][6], sb[i][7]);
        } else {
          w.x = __float_as_uint(sb[i][0]);
          w.y = __float_as_uint(sb[i][1]);
          w.z = __float_as_uint(sb[i][2]);
          w.w = __float_as_uint(sb[i][3]);
        }
        *reinterpret_cast<uint4*>(bp + (r0 + RPP * i) * K + c0) = w;
      }
    }
  }
}

template <bool BF16, bool ALIGN>
static hipError_t launch_q(const CommitParams& p, int window, dim3 grid, hipStream_t stream) {
  switch (window) {
#define KDA_COMMIT_CASE(QQ)                                                                \
  case QQ:                                                                                \
    hipLaunchKernelGGL((commit_kernel<BF16, QQ, ALIGN>), grid, dim3(256), 0, stream, p); \
    break;
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
  if (bf16) return align ? launch_q<true, true>(p, window, grid, stream)
                         : launch_q<true, false>(p, window, grid, stream);
  return align ? launch_q<false, true>(p, window, grid, stream)
               : launch_q<false, false>(p, window, grid, stream);
}

}  // namespace kda
