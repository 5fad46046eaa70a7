/*
 * KDA gated delta-rule oracle: a plain, sequential, FP64 CPU implementation of
 * everything the GPU library computes.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The GPU library neither links nor calls it,
 * and the two share no source, header, table or helper.
 *
 * Sources are the vLLM API pages on Kimi-K3 KDA, cited by page title:
 *   [commit page]  vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.commit
 *   [kernels page] vllm.models.kimi_k3.nvidia.specialized_decode.recoverssm.kernels
 *   [fused page]   vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.fused
 *
 * Precision: every input is converted exactly to double (BF16 and FP32 are
 * subsets of FP64); all arithmetic is FP64 in the order the definitions give;
 * each stored output is rounded once, round-to-nearest-even, to its dtype. The
 * one exception is the convolution prologue's SiLU, whose BF16 rounding is a
 * decision taken in FP32 by fixed steps (see "Convolution prologue").
 *
 * Shapes are runtime parameters (K key channels, V value channels) so that the
 * same code runs at K = V = 128 and on tiny brute-force cases.
 *
 * Parity pins (what checks this file against something other than itself) live
 * in tests/test_oracle_*.py; the check-only forms below (closed-form commit,
 * log-space commit, chunked WY verify) exist only for those pins.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Scalar conversions                                                         */
/* ------------------------------------------------------------------------- */

double kda_o_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round a double straight to BF16 (8 significant bits), ties to even, with no
 * intermediate FP32 rounding (which would round twice). */
uint16_t kda_o_double_to_bf16(double x) {
  if (isnan(x)) return (uint16_t)0x7fc0;
  double ax = fabs(x);
  uint16_t sign = signbit(x) ? (uint16_t)0x8000 : (uint16_t)0;
  if (ax == 0.0) return sign;
  if (isinf(x)) return (uint16_t)(sign | 0x7f80);
  int e;
  frexp(ax, &e); /* ax = m * 2^e, 0.5 <= m < 1 */
  /* The unit in the last place: 2^(e-8) for normals, 2^-133 below 2^-126. */
  int ulp_exp = e - 8;
  if (ulp_exp < -133) ulp_exp = -133;
  double scaled = ldexp(ax, -ulp_exp);  /* exact: a power-of-two scale */
  double r = nearbyint(scaled);         /* default mode: ties to even */
  double y = ldexp(r, ulp_exp);         /* exactly representable in BF16 */
  if (y > 3.3895313892515355e38) return (uint16_t)(sign | 0x7f80);
  float f = (float)y; /* exact */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7fff));
}

static float to_f32(double x) { return (float)x; }

/* ------------------------------------------------------------------------- */
/* The method's scalar and vector steps                                       */
/* ------------------------------------------------------------------------- */

/* Bounded KDA gate decay, [fused page] KdaFused.decay:
 *   d = exp(lb * sigmoid(exp(A_log) * (g + dt_bias))),  sigmoid(x) = 1/(1+e^-x). */
double kda_o_decay(double g, double a_log, double dt_bias, double lower_bound) {
  double z = exp(a_log) * (g + dt_bias);
  double sig = 1.0 / (1.0 + exp(-z));
  return exp(lower_bound * sig);
}

/* beta = sigmoid(raw_beta), [fused page] KdaFused.kernel (the beta operand). */
double kda_o_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Key L2 normalisation with 1e-6 inside the root, applied at every use of a key:
 * [commit page] KdaCommit.kernel (recorded keys), [fused page] KdaFused.kernel
 * (new and recorded keys). */
void kda_o_knorm(int K, const double* k, double* out) {
  double s = 0.0;
  for (int c = 0; c < K; ++c) s += k[c] * k[c];
  double inv = 1.0 / sqrt(s + 1e-6);
  for (int c = 0; c < K; ++c) out[c] = k[c] * inv;
}

/* ------------------------------------------------------------------------- */
/* Convolution prologue ([fused page] KdaFused.kernel: the convolution, its    */
/* SiLU, and the q/k normalisation)                                           */
/* ------------------------------------------------------------------------- */
/*
 * The SiLU output is stored in BF16 and is then used everywhere (the recorded
 * key is its bit pattern). Its BF16 rounding is therefore a decision that both
 * sides must take identically, and it is taken in FP32, the page's precision,
 * by these fixed steps (the GPU kernel implements the same steps on its own):
 *   acc = bias; acc = fma(seq_{t+i}, w_i, acc) for i = 0, 1, 2, 3;
 *   e   = exp_f32(-acc)   (below);
 *   y   = BF16_rne(acc / (1 + e))   (IEEE FP32 add and divide).
 * Everything after the rounding is FP64 again.
 */

/* exp in FP32 by Cody and Waite's two-constant argument reduction and a
 * degree-7 Taylor polynomial (Horner form, each step one fused multiply-add):
 *   x is clamped to [-80, 80];  k = rint(x * log2(e));
 *   r = fma(-k, LN2_HI, x);  r = fma(-k, LN2_LO, r);
 *   p = 1 + r + r^2/2! + ... + r^7/7!;  exp(x) = p * 2^k.
 * LN2_HI is ln 2 rounded to 16 fraction bits (so k * LN2_HI is exact for
 * |k| < 256), LN2_LO the FP32 value of ln 2 - LN2_HI; the Taylor coefficients
 * are the FP32 quotients 1/j!. Error: |r| <= ln2/2, so the truncation is below
 * 2e-9 relative, and the result is within a few FP32 ulps of exp(x). */
static const float kda_o_ln2_hi = 45426.0f / 65536.0f;

float kda_o_exp_f32(float x) {
  const float ln2_lo = (float)(0.69314718055994530942 - (double)kda_o_ln2_hi);
  const float log2e = 1.44269504088896340736f;
  float c[8];
  float f = 1.0f;
  for (int j = 0; j < 8; ++j) {
    if (j > 1) f *= (float)j; /* j! is exact in FP32 for j <= 7 */
    c[j] = 1.0f / f;
  }
  if (x > 80.0f) x = 80.0f;
  if (x < -80.0f) x = -80.0f;
  float k = rintf(x * log2e);
  float r = fmaf(-k, kda_o_ln2_hi, x);
  r = fmaf(-k, ln2_lo, r);
  float p = c[7];
  for (int j = 6; j >= 0; --j) p = fmaf(p, r, c[j]);
  return ldexpf(p, (int)k);
}

/* SiLU of an FP32 pre-activation, rounded to BF16 (the steps above). */
uint16_t kda_o_silu_bf16(float acc) {
  float e = kda_o_exp_f32(-acc);
  float y = acc / (1.0f + e);
  return kda_o_double_to_bf16((double)y);
}

/* One channel's causal convolution over a window of T tokens: seq holds the 3
 * history taps then the T inputs (BF16 values), w the 4 weights (w[0] meets the
 * oldest tap, w[3] the current input), bias 0 when there is none. Writes the
 * BF16 bits of SiLU(bias + sum_i w_i seq_{t+i}) for t < T. */
void kda_o_conv_silu(int T, const float* seq, const float* w, float bias, uint16_t* y) {
  for (int t = 0; t < T; ++t) {
    float acc = bias;
    for (int i = 0; i < 4; ++i) acc = fmaf(seq[t + i], w[i], acc);
    y[t] = kda_o_silu_bf16(acc);
  }
}

/* ------------------------------------------------------------------------- */
/* Low-rank gate projection ([fused page] KdaFused.kernel, the gate           */
/* projection)                                                                */
/* ------------------------------------------------------------------------- */

/* raw_g[t][f] = BF16(sum_j F_A[t][j] * F_B[f][j]), j < R (R = 128 on the page):
 * F_A row t at f_a + t * sa (BF16 bits), F_B row f at f_b + f * R, out row t at
 * out + t * D. FP64 sum, rounded once. */
void kda_o_gate_projection(long N, int D, int R, const uint16_t* f_a, int64_t sa,
                           const uint16_t* f_b, uint16_t* out) {
  for (long t = 0; t < N; ++t)
    for (int f = 0; f < D; ++f) {
      double acc = 0.0;
      for (int j = 0; j < R; ++j)
        acc += kda_o_bf16_to_double(f_a[t * sa + j]) *
               kda_o_bf16_to_double(f_b[(int64_t)f * R + j]);
      out[t * (int64_t)D + f] = kda_o_double_to_bf16(acc);
    }
}

/* The window offset of a fused step: the history after n accepted tokens of the
 * previous window starts at n - 1 (at 0 when nothing is pending). */
int kda_o_conv_offset(int n) { return n > 0 ? n - 1 : 0; }

/* ------------------------------------------------------------------------- */
/* Item-level cores (double in, double out). Layouts: S is [V][K] row-major   */
/* (row v = value channel, column c = key channel); per-token vectors are     */
/* [T][K] or [T][V].                                                          */
/* ------------------------------------------------------------------------- */

/* RecoverSSM commit, sequential form: replay the recorded tokens one at a time,
 *   S <- S diag(d_t) + u_t kn_t^T   for t < n,
 * with the recorded corrections u_t (not recomputed). This is the stock
 * recurrence's state update ([fused page] module docstring) with u_t given. */
void kda_o_commit_seq(int K, int V, int n, const double* S0, const double* u,
                      const double* kn, const double* d, double* S) {
  memcpy(S, S0, sizeof(double) * (size_t)V * (size_t)K);
  for (int t = 0; t < n; ++t)
    for (int v = 0; v < V; ++v)
      for (int c = 0; c < K; ++c)
        S[v * K + c] = S[v * K + c] * d[t * K + c] + u[t * V + v] * kn[t * K + c];
}

/* CHECK-ONLY. Closed form of the commit ([commit page] module docstring,
 * [fused page] module docstring, step 1):
 *   S_n = S_0 diag(D_n) + sum_{t<n} u_t (kn_t * P_t)^T,
 *   D_n = prod_{s<n} d_s,  P_t = prod_{t<s<n} d_s. */
void kda_o_commit_closed(int K, int V, int n, const double* S0, const double* u,
                         const double* kn, const double* d, double* S) {
  double* D = (double*)malloc(sizeof(double) * (size_t)K);
  double* P = (double*)malloc(sizeof(double) * (size_t)K);
  for (int c = 0; c < K; ++c) {
    D[c] = 1.0;
    for (int s = 0; s < n; ++s) D[c] *= d[s * K + c];
  }
  for (int v = 0; v < V; ++v)
    for (int c = 0; c < K; ++c) S[v * K + c] = S0[v * K + c] * D[c];
  for (int t = 0; t < n; ++t) {
    for (int c = 0; c < K; ++c) {
      P[c] = 1.0;
      for (int s = t + 1; s < n; ++s) P[c] *= d[s * K + c];
    }
    for (int v = 0; v < V; ++v)
      for (int c = 0; c < K; ++c) S[v * K + c] += u[t * V + v] * (kn[t * K + c] * P[c]);
  }
  free(D);
  free(P);
}

/* CHECK-ONLY. The commit in the log space the commit kernel uses
 * ([commit page] KdaCommit.kernel): with L_t = sum_{s<=t} log d_s,
 * D_n = exp(L_{n-1}) and P_t = exp(L_{n-1} - L_t). */
void kda_o_commit_logspace(int K, int V, int n, const double* S0, const double* u,
                           const double* kn, const double* d, double* S) {
  double* L = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)K);
  for (int c = 0; c < K; ++c) {
    double cum = 0.0;
    for (int t = 0; t < n; ++t) {
      cum += log(d[t * K + c]);
      L[t * K + c] = cum;
    }
  }
  for (int v = 0; v < V; ++v)
    for (int c = 0; c < K; ++c) {
      double last = n > 0 ? L[(n - 1) * K + c] : 0.0;
      double acc = S0[v * K + c] * exp(last);
      for (int t = 0; t < n; ++t)
        acc += u[t * V + v] * (kn[t * K + c] * exp(last - L[t * K + c]));
      S[v * K + c] = acc;
    }
  free(L);
}

/* The stock gated delta-rule recurrence ([fused page] module docstring, the
 * recurrence the chunked form rewrites), one token at a time:
 *   S <- S diag(d_t);  u_t = beta_t (v_t - S kn_t);  S <- S + u_t kn_t^T;  o_t = S q_t.
 * S is updated in place and holds the state after the last token on return. */
void kda_o_verify_seq(int K, int V, int T, double* S, const double* q, const double* kn,
                      const double* vv, const double* d, const double* beta, double* o,
                      double* u) {
  for (int t = 0; t < T; ++t) {
    for (int v = 0; v < V; ++v)
      for (int c = 0; c < K; ++c) S[v * K + c] *= d[t * K + c];
    for (int v = 0; v < V; ++v) {
      double sk = 0.0;
      for (int c = 0; c < K; ++c) sk += S[v * K + c] * kn[t * K + c];
      u[t * V + v] = beta[t] * (vv[t * V + v] - sk);
    }
    for (int v = 0; v < V; ++v)
      for (int c = 0; c < K; ++c) S[v * K + c] += u[t * V + v] * kn[t * K + c];
    for (int v = 0; v < V; ++v) {
      double sq = 0.0;
      for (int c = 0; c < K; ++c) sq += S[v * K + c] * q[t * K + c];
      o[t * V + v] = sq;
    }
  }
}

/* CHECK-ONLY. The chunked (WY) verify from an unmodified S ([fused page] module
 * docstring, step 2): with Gamma_t = prod_{r<=t} d_r and P(s,t) = prod_{s<r<=t} d_r,
 *   w_t = S (Gamma_t * kn_t),  y_t = S (Gamma_t * q_t),
 *   A_ts = kn_s . (P(s,t) * kn_t)  (s < t),  B_ts = kn_s . (P(s,t) * q_t)  (s <= t),
 *   u_t = beta_t (v_t - w_t - sum_{s<t} A_ts u_s),  o_t = y_t + sum_{s<=t} B_ts u_s. */
void kda_o_verify_wy(int K, int V, int T, const double* S, const double* q, const double* kn,
                     const double* vv, const double* d, const double* beta, double* o,
                     double* u) {
  double* G = (double*)malloc(sizeof(double) * (size_t)T * (size_t)K);
  double* A = (double*)calloc((size_t)T * (size_t)T, sizeof(double));
  double* Bm = (double*)calloc((size_t)T * (size_t)T, sizeof(double));
  double* w = (double*)malloc(sizeof(double) * (size_t)T * (size_t)V);
  double* y = (double*)malloc(sizeof(double) * (size_t)T * (size_t)V);
  for (int c = 0; c < K; ++c) {
    double g = 1.0;
    for (int t = 0; t < T; ++t) {
      g *= d[t * K + c];
      G[t * K + c] = g;
    }
  }
  for (int t = 0; t < T; ++t)
    for (int v = 0; v < V; ++v) {
      double sw = 0.0, sy = 0.0;
      for (int c = 0; c < K; ++c) {
        sw += S[v * K + c] * (G[t * K + c] * kn[t * K + c]);
        sy += S[v * K + c] * (G[t * K + c] * q[t * K + c]);
      }
      w[t * V + v] = sw;
      y[t * V + v] = sy;
    }
  for (int t = 0; t < T; ++t)
    for (int s = 0; s <= t; ++s) {
      double sa = 0.0, sb = 0.0;
      for (int c = 0; c < K; ++c) {
        double p = 1.0;
        for (int r = s + 1; r <= t; ++r) p *= d[r * K + c];
        sa += kn[s * K + c] * (p * kn[t * K + c]);
        sb += kn[s * K + c] * (p * q[t * K + c]);
      }
      if (s < t) A[t * T + s] = sa;
      Bm[t * T + s] = sb;
    }
  for (int v = 0; v < V; ++v)
    for (int t = 0; t < T; ++t) {
      double acc = vv[t * V + v] - w[t * V + v];
      for (int s = 0; s < t; ++s) acc -= A[t * T + s] * u[s * V + v];
      u[t * V + v] = beta[t] * acc;
      double oo = y[t * V + v];
      for (int s = 0; s <= t; ++s) oo += Bm[t * T + s] * u[s * V + v];
      o[t * V + v] = oo;
    }
  free(G);
  free(A);
  free(Bm);
  free(w);
  free(y);
}

/* ------------------------------------------------------------------------- */
/* A minimal work queue over items (one pthread per worker).                  */
/* ------------------------------------------------------------------------- */

typedef void (*item_fn)(void* ctx, long item);
struct pool {
  item_fn fn;
  void* ctx;
  long count;
  long next; /* atomic */
};

static void* pool_worker(void* p) {
  struct pool* w = (struct pool*)p;
  for (;;) {
    long i = __atomic_fetch_add(&w->next, 1, __ATOMIC_RELAXED);
    if (i >= w->count) break;
    w->fn(w->ctx, i);
  }
  return NULL;
}

static void parallel_for(long count, int threads, item_fn fn, void* ctx) {
  struct pool w = {fn, ctx, count, 0};
  if (threads > 256) threads = 256;
  if (threads <= 1 || count < 2) {
    pool_worker(&w);
    return;
  }
  pthread_t tid[256];
  int started = 0;
  for (int t = 0; t < threads; ++t) {
    if (pthread_create(&tid[t], NULL, pool_worker, &w) != 0) break;
    ++started;
  }
  if (started == 0) pool_worker(&w);
  for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
}

/* ------------------------------------------------------------------------- */
/* Buffer-level operations with the library's semantics, on host buffers.     */
/* ------------------------------------------------------------------------- */

/* kda_commit ([commit page] module and class docstrings, KdaCommit.kernel).
 * Items are (layer, request, head). An item is live when n > 0, source > null,
 * destination > null and its record row >= 0; then
 *   destination page <- commit of min(n, Q) recorded tokens onto the source page,
 *   boundary page    <- commit of min(m, min(n, Q)) tokens (when m > 0 and
 *                       boundary > null; align only).
 * A non-live item writes nothing. The record row is record_rows[b] when given,
 * else b. Records hold Q tokens per head: corrections [rows][H][Q][V] FP32,
 * key/gate [rows][H][Q][2K] BF16 (raw key, then raw gate). */
struct commit_ctx {
  int L, H, Q, B, K, V, bf16;
  void* const* state;
  const int64_t* state_stride;
  const float* const* corr;
  const int64_t* corr_stride;
  const uint16_t* const* kg;
  const int64_t* kg_stride;
  const float* a_log;
  const float* dt_bias;
  const int32_t* sources;
  const int32_t* lens;
  const int32_t* dests;
  const int32_t* bounds;
  const int32_t* blens;
  const int32_t* rows;
  double lb;
  int null_slot;
  const int64_t* items; /* optional subset (flattened item ids) */
};

static double state_get(const void* base, int bf16, int64_t idx) {
  if (bf16) return kda_o_bf16_to_double(((const uint16_t*)base)[idx]);
  return (double)((const float*)base)[idx];
}

static void state_put(void* base, int bf16, int64_t idx, double x) {
  if (bf16)
    ((uint16_t*)base)[idx] = kda_o_double_to_bf16(x);
  else
    ((float*)base)[idx] = to_f32(x);
}

static void commit_item(void* p, long it) {
  const struct commit_ctx* c = (const struct commit_ctx*)p;
  long item = c->items ? (long)c->items[it] : it;
  int K = c->K, V = c->V, Q = c->Q;
  int h = (int)(item % c->H);
  int b = (int)((item / c->H) % c->B);
  int l = (int)(item / ((long)c->H * c->B));
  int n = c->lens[b];
  int src = c->sources[b], dst = c->dests[b];
  int row = c->rows ? c->rows[b] : b;
  if (!(n > 0 && src > c->null_slot && dst > c->null_slot && row >= 0)) return;
  int m = 0, bnd = c->null_slot;
  if (c->bounds && c->blens) {
    m = c->blens[b];
    bnd = c->bounds[b];
  }
  int boundary_live = m > 0 && bnd > c->null_slot;
  int ne = n < Q ? n : Q;
  int me = m < ne ? m : ne;

  size_t VK = (size_t)V * (size_t)K;
  double* S0 = (double*)malloc(sizeof(double) * VK);
  double* S = (double*)malloc(sizeof(double) * VK);
  double* u = (double*)malloc(sizeof(double) * (size_t)Q * V);
  double* kn = (double*)malloc(sizeof(double) * (size_t)Q * K);
  double* d = (double*)malloc(sizeof(double) * (size_t)Q * K);
  double* kr = (double*)malloc(sizeof(double) * (size_t)K);

  const void* base = c->state[l];
  int64_t src_off = (int64_t)src * c->state_stride[l] + (int64_t)h * (int64_t)VK;
  for (size_t i = 0; i < VK; ++i) S0[i] = state_get(base, c->bf16, src_off + (int64_t)i);

  const float* corr = c->corr[l] + (int64_t)row * c->corr_stride[l] + (int64_t)h * Q * V;
  const uint16_t* kg = c->kg[l] + (int64_t)row * c->kg_stride[l] + (int64_t)h * Q * 2 * K;
  double a = c->a_log[l * c->H + h];
  const float* dtb = c->dt_bias + ((int64_t)l * c->H + h) * K;
  for (int t = 0; t < ne; ++t) {
    for (int v = 0; v < V; ++v) u[t * V + v] = (double)corr[t * V + v];
    for (int ch = 0; ch < K; ++ch) {
      kr[ch] = kda_o_bf16_to_double(kg[t * 2 * K + ch]);
      double g = kda_o_bf16_to_double(kg[t * 2 * K + K + ch]);
      d[t * K + ch] = kda_o_decay(g, a, (double)dtb[ch], c->lb);
    }
    kda_o_knorm(K, kr, kn + t * K);
  }

  void* out = c->state[l];
  if (boundary_live) {
    kda_o_commit_seq(K, V, me, S0, u, kn, d, S);
    int64_t off = (int64_t)bnd * c->state_stride[l] + (int64_t)h * (int64_t)VK;
    for (size_t i = 0; i < VK; ++i) state_put(out, c->bf16, off + (int64_t)i, S[i]);
  }
  kda_o_commit_seq(K, V, ne, S0, u, kn, d, S);
  int64_t off = (int64_t)dst * c->state_stride[l] + (int64_t)h * (int64_t)VK;
  for (size_t i = 0; i < VK; ++i) state_put(out, c->bf16, off + (int64_t)i, S[i]);

  free(S0);
  free(S);
  free(u);
  free(kn);
  free(d);
  free(kr);
}

int kda_o_commit(int L, int H, int Q, int B, int K, int V, int state_bf16,
                 void* const* state_addrs, const int64_t* state_slot_strides,
                 const float* const* corr_addrs, const int64_t* corr_row_strides,
                 const uint16_t* const* kg_addrs, const int64_t* kg_row_strides,
                 const float* a_log, const float* dt_bias, const int32_t* sources,
                 const int32_t* commit_lens, const int32_t* destinations,
                 const int32_t* boundaries, const int32_t* boundary_lens,
                 const int32_t* record_rows, double lower_bound, int null_slot,
                 const int64_t* items, long n_items, int threads) {
  struct commit_ctx c = {L,     H,       Q,      B,           K,          V,
                         state_bf16, state_addrs, state_slot_strides, corr_addrs, corr_row_strides,
                         kg_addrs,   kg_row_strides, a_log, dt_bias, sources, commit_lens,
                         destinations, boundaries, boundary_lens, record_rows, lower_bound,
                         null_slot, items};
  long count = items ? n_items : (long)L * B * H;
  parallel_for(count, threads, commit_item, &c);
  return 0;
}

/* kda_verify / kda_fused_replay_verify ([kernels page] kda_recoverssm_verify;
 * [fused page] module docstring and KdaFused.kernel). Items are (request, head).
 *  - the item's window: rows tok0 + t, t < L, with tok0 = b*T and L = T, or
 *    (query_start_loc given) tok0 = qsl[b], L = clamp(qsl[b+1] - qsl[b], 0, T);
 *    L = 0 is padding: nothing is read or written.
 *  - state slot <= null: the item's L x V outputs are zero; nothing else.
 *  - record row rec = record_rows[b] (or b when record_rows is NULL).
 *  - fused only: n = clamp(pending[rec], 0, RQ) when rec >= 0, else 0; the n
 *    recorded tokens are replayed onto S_0 and S_n is written back when n > 0.
 *    With boundaries (align, as the commit's): when n > 0, bnd = bounds[b] >
 *    null and m = blens[b] > 0, S_{min(m, n)} is also stored to slot bnd.
 *  - the stock recurrence runs over the L new tokens from S_n (verify: S_0);
 *    o -> BF16 out[tok0 + t][h*V + v].
 *  - rec >= 0: the records of tokens t < L are rewritten (u_t FP32, raw key and
 *    raw gate bit copies), after every old record of the item was read.
 * q is used as given; keys are normalised; beta = sigmoid(raw_beta). */
struct verify_ctx {
  int H, T, B, K, V, RQ, fused, state_bf16;
  const uint16_t *q, *k, *v, *g, *rb;
  const float* a_log;
  const float* dt_bias;
  double lb;
  void* state; /* FP32 or BF16 pool */
  int64_t slot_stride;
  const int32_t* slots;
  int null_slot;
  float* corr;
  uint16_t* kg;
  const int32_t* rows;
  const int32_t* pending;
  uint16_t* out;
  const int64_t* items;
  const uint16_t* gate;  /* optional gated RMSNorm epilogue */
  const float* norm_w;
  double norm_eps;
  const int32_t* qsl;     /* optional [B+1] token offsets (variable-length windows) */
  const int32_t* bounds;  /* fused, optional: boundary slots [B] (align) */
  const int32_t* blens;   /*   and boundary lengths m [B] */
  /* optional convolution prologue (x != NULL): q, k, v are its outputs */
  const uint16_t* x;      /* [B*T] rows of x_stride: q | k | v pre-activations */
  int64_t x_stride;
  const uint16_t* conv_w; /* BF16 [3][4][H*K] */
  const uint16_t* conv_b; /* BF16 [3*H*K] or NULL */
  uint16_t* conv;         /* BF16 window pool */
  int64_t conv_ss, conv_cs, conv_ts; /* slot, channel, tap strides (elements) */
  double q_scale;
  double* o_raw;          /* optional: o before any rounding, laid out as out (a check aid) */
};

/* The prologue of one item: per part p (0 q, 1 k, 2 v) and channel, the window
 * taps at the replay-aware offset, the convolution and SiLU of the T inputs, and
 * the window write-back [tap 1, tap 2, x_0 .. x_{T-1}] (entries past T + 1 keep
 * their values). y is [3][T][K] BF16 bits. */
static void conv_prologue(const struct verify_ctx* c, int b, int h, int slot, int n,
                          uint16_t* y) {
  const int K = c->K, T = c->T, d = c->H * c->K;
  const int off = kda_o_conv_offset(n);
  float seq[3 + 8];
  float w[4];
  uint16_t yt[8];
  for (int p = 0; p < 3; ++p) {
    for (int ch = 0; ch < K; ++ch) {
      const int64_t col = (int64_t)p * d + (int64_t)h * K + ch;
      uint16_t* win = c->conv + (int64_t)slot * c->conv_ss + col * c->conv_cs;
      uint16_t taps[3];
      for (int i = 0; i < 3; ++i) taps[i] = win[(int64_t)(off + i) * c->conv_ts];
      for (int i = 0; i < 3; ++i) seq[i] = (float)kda_o_bf16_to_double(taps[i]);
      uint16_t xin[8];
      for (int t = 0; t < T; ++t) {
        xin[t] = c->x[((int64_t)b * T + t) * c->x_stride + col];
        seq[3 + t] = (float)kda_o_bf16_to_double(xin[t]);
      }
      for (int i = 0; i < 4; ++i)
        w[i] = (float)kda_o_bf16_to_double(c->conv_w[((int64_t)p * 4 + i) * d + (int64_t)h * K + ch]);
      float bias = c->conv_b ? (float)kda_o_bf16_to_double(c->conv_b[col]) : 0.0f;
      kda_o_conv_silu(T, seq, w, bias, yt);
      for (int t = 0; t < T; ++t) y[((int64_t)p * T + t) * K + ch] = yt[t];
      /* write-back, after this channel's window was read */
      win[0] = taps[1];
      win[c->conv_ts] = taps[2];
      for (int t = 0; t < T; ++t) win[(int64_t)(2 + t) * c->conv_ts] = xin[t];
    }
  }
}

/* Gated RMSNorm of one token's outputs ([fused page] KdaFused.kernel, the
 * output stage): o is first rounded to BF16 (a stock rounding point); then
 * rstd = 1 / sqrt(mean_v(o_bf^2) + eps) and out = o_bf * rstd * w[v] * sigmoid(gate[v]). */
static void gated_rmsnorm(int V, const double* o, const uint16_t* gate, const float* w,
                          double eps, uint16_t* out) {
  double ss = 0.0;
  for (int v = 0; v < V; ++v) {
    double ob = kda_o_bf16_to_double(kda_o_double_to_bf16(o[v]));
    ss += ob * ob;
  }
  double rstd = 1.0 / sqrt(ss / (double)V + eps);
  for (int v = 0; v < V; ++v) {
    double ob = kda_o_bf16_to_double(kda_o_double_to_bf16(o[v]));
    double gv = kda_o_sigmoid(kda_o_bf16_to_double(gate[v]));
    out[v] = kda_o_double_to_bf16(ob * rstd * (double)w[v] * gv);
  }
}

static void verify_item(void* p, long it) {
  const struct verify_ctx* c = (const struct verify_ctx*)p;
  long item = c->items ? (long)c->items[it] : it;
  int K = c->K, V = c->V, T = c->T, H = c->H, RQ = c->RQ;
  int h = (int)(item % H);
  int b = (int)(item / H);
  /* The item's tokens: rows tok0 .. tok0 + T - 1, with T its window length
   * (query_start_loc: qsl[b+1] - qsl[b], clamped to 0..T). An empty window is
   * padding: nothing is read or written. */
  int64_t tok0 = (int64_t)b * T;
  if (c->qsl) {
    tok0 = c->qsl[b];
    int L = c->qsl[b + 1] - c->qsl[b];
    T = L < 0 ? 0 : (L > T ? T : L);
  }
  if (T == 0) return;
  int slot = c->slots[b];
  if (slot <= c->null_slot) {
    for (int t = 0; t < T; ++t)
      for (int v = 0; v < V; ++v) {
        c->out[(tok0 + t) * H * V + (int64_t)h * V + v] = kda_o_double_to_bf16(0.0);
        if (c->o_raw) c->o_raw[(tok0 + t) * H * V + (int64_t)h * V + v] = 0.0;
      }
    return;
  }
  int rec = c->rows ? c->rows[b] : b;
  int n = 0;
  if (c->fused && rec >= 0) {
    n = c->pending[rec];
    if (n > RQ) n = RQ;
    if (n < 0) n = 0;
  }
  size_t VK = (size_t)V * (size_t)K;
  double* S0 = (double*)malloc(sizeof(double) * VK);
  double* S = (double*)malloc(sizeof(double) * VK);
  int TM = T > RQ ? T : RQ;
  double* u = (double*)malloc(sizeof(double) * (size_t)TM * V);
  double* kn = (double*)malloc(sizeof(double) * (size_t)TM * K);
  double* d = (double*)malloc(sizeof(double) * (size_t)TM * K);
  double* qq = (double*)malloc(sizeof(double) * (size_t)T * K);
  double* vv = (double*)malloc(sizeof(double) * (size_t)T * V);
  double* beta = (double*)malloc(sizeof(double) * (size_t)T);
  double* o = (double*)malloc(sizeof(double) * (size_t)T * V);
  double* kr = (double*)malloc(sizeof(double) * (size_t)K);

  const int64_t page = (int64_t)slot * c->slot_stride + (int64_t)h * (int64_t)VK;
  for (size_t i = 0; i < VK; ++i) S0[i] = state_get(c->state, c->state_bf16, page + (int64_t)i);
  double a = c->a_log[h];
  const float* dtb = c->dt_bias + (int64_t)h * K;

  /* Replay of the pending tokens from the old records (all read here, before
   * any record is rewritten below). */
  if (n > 0) {
    const float* corr = c->corr + (((int64_t)rec * H + h) * RQ) * V;
    const uint16_t* kg = c->kg + (((int64_t)rec * H + h) * RQ) * 2 * K;
    for (int t = 0; t < n; ++t) {
      for (int v = 0; v < V; ++v) u[t * V + v] = (double)corr[t * V + v];
      for (int ch = 0; ch < K; ++ch) {
        kr[ch] = kda_o_bf16_to_double(kg[t * 2 * K + ch]);
        double gg = kda_o_bf16_to_double(kg[t * 2 * K + K + ch]);
        d[t * K + ch] = kda_o_decay(gg, a, (double)dtb[ch], c->lb);
      }
      kda_o_knorm(K, kr, kn + t * K);
    }
    if (c->bounds && c->blens && c->bounds[b] > c->null_slot && c->blens[b] > 0) {
      const int me = c->blens[b] < n ? c->blens[b] : n;
      kda_o_commit_seq(K, V, me, S0, u, kn, d, S);
      const int64_t bpage = (int64_t)c->bounds[b] * c->slot_stride + (int64_t)h * (int64_t)VK;
      for (size_t i = 0; i < VK; ++i)
        state_put(c->state, c->state_bf16, bpage + (int64_t)i, S[i]);
    }
    kda_o_commit_seq(K, V, n, S0, u, kn, d, S);
    for (size_t i = 0; i < VK; ++i) state_put(c->state, c->state_bf16, page + (int64_t)i, S[i]);
  } else {
    memcpy(S, S0, sizeof(double) * VK);
  }

  /* The new window: q, k, v given, or the convolution prologue's outputs (then
   * q is L2-normalised with 1e-6 inside the root and scaled by q_scale). */
  uint16_t* ycv = NULL;
  if (c->x) {
    ycv = (uint16_t*)malloc(sizeof(uint16_t) * 3 * (size_t)T * (size_t)K);
    conv_prologue(c, b, h, slot, n, ycv);
  }
  for (int t = 0; t < T; ++t) {
    int64_t tok = tok0 + t;
    const uint16_t* qt = ycv ? ycv + (0 * T + t) * K : c->q + (tok * H + h) * K;
    const uint16_t* kt = ycv ? ycv + (1 * T + t) * K : c->k + (tok * H + h) * K;
    const uint16_t* vt = ycv ? ycv + (2 * T + t) * K : c->v + (tok * H + h) * V;
    const uint16_t* gt = c->g + (tok * H + h) * K;
    for (int ch = 0; ch < K; ++ch) {
      qq[t * K + ch] = kda_o_bf16_to_double(qt[ch]);
      kr[ch] = kda_o_bf16_to_double(kt[ch]);
      d[t * K + ch] = kda_o_decay(kda_o_bf16_to_double(gt[ch]), a, (double)dtb[ch], c->lb);
    }
    if (ycv) {
      double sq = 0.0;
      for (int ch = 0; ch < K; ++ch) sq += qq[t * K + ch] * qq[t * K + ch];
      double f = c->q_scale / sqrt(sq + 1e-6);
      for (int ch = 0; ch < K; ++ch) qq[t * K + ch] *= f;
    }
    kda_o_knorm(K, kr, kn + t * K);
    for (int v = 0; v < V; ++v) vv[t * V + v] = kda_o_bf16_to_double(vt[v]);
    beta[t] = kda_o_sigmoid(kda_o_bf16_to_double(c->rb[tok * H + h]));
  }
  kda_o_verify_seq(K, V, T, S, qq, kn, vv, d, beta, o, u);

  for (int t = 0; t < T; ++t) {
    uint16_t* orow = c->out + (tok0 + t) * H * V + (int64_t)h * V;
    if (c->o_raw)
      for (int v = 0; v < V; ++v) c->o_raw[(tok0 + t) * H * V + (int64_t)h * V + v] = o[t * V + v];
    if (c->gate && c->norm_w) {
      gated_rmsnorm(V, o + t * V, c->gate + (tok0 + t) * H * V + (int64_t)h * V,
                    c->norm_w, c->norm_eps, orow);
    } else {
      for (int v = 0; v < V; ++v) orow[v] = kda_o_double_to_bf16(o[t * V + v]);
    }
  }
  if (rec >= 0) {
    float* corr = c->corr + (((int64_t)rec * H + h) * RQ) * V;
    uint16_t* kg = c->kg + (((int64_t)rec * H + h) * RQ) * 2 * K;
    for (int t = 0; t < T; ++t) {
      int64_t tok = tok0 + t;
      for (int v = 0; v < V; ++v) corr[t * V + v] = to_f32(u[t * V + v]);
      for (int ch = 0; ch < K; ++ch) {
        kg[t * 2 * K + ch] = ycv ? ycv[(1 * T + t) * K + ch] : c->k[(tok * H + h) * K + ch];
        kg[t * 2 * K + K + ch] = c->g[(tok * H + h) * K + ch];
      }
    }
  }
  free(ycv);
  free(S0);
  free(S);
  free(u);
  free(kn);
  free(d);
  free(qq);
  free(vv);
  free(beta);
  free(o);
  free(kr);
}

int kda_o_verify(int H, int T, int B, int K, int V, const uint16_t* q, const uint16_t* k,
                 const uint16_t* v, const uint16_t* raw_g, const uint16_t* raw_beta,
                 const float* a_log, const float* dt_bias, double lower_bound, void* state,
                 int64_t state_slot_stride, const int32_t* state_indices, int null_slot,
                 float* corr, uint16_t* kg, int RQ, const int32_t* record_rows,
                 const int32_t* pending, int fused, uint16_t* out, const int64_t* items,
                 long n_items, int threads, const uint16_t* gate, const float* norm_w,
                 double norm_eps, int state_bf16, const uint16_t* x, int64_t x_stride,
                 const uint16_t* conv_w, const uint16_t* conv_b, uint16_t* conv,
                 int64_t conv_ss, int64_t conv_cs, int64_t conv_ts, double q_scale,
                 const int32_t* query_start_loc, const int32_t* boundaries,
                 const int32_t* boundary_lens, double* o_raw) {
  struct verify_ctx c = {H,          T,          B,       K,          V,
                         RQ,         fused,      state_bf16, q,       k,          v,
                         raw_g,      raw_beta,   a_log,   dt_bias,    lower_bound,
                         state,      state_slot_stride, state_indices, null_slot, corr,
                         kg,         record_rows, pending, out,       items,
                         gate,       norm_w,     norm_eps, query_start_loc, boundaries,
                         boundary_lens, x, x_stride,
                         conv_w,     conv_b,     conv,    conv_ss,    conv_cs,
                         conv_ts,    q_scale,    o_raw};
  long count = items ? n_items : (long)B * H;
  parallel_for(count, threads, verify_item, &c);
  return 0;
}

/* kda_decay over a [N][H][K] BF16 raw-gate tensor -> FP32 ([fused page]
 * KdaFused.decay). */
void kda_o_decay_buf(long N, int H, int K, const uint16_t* raw_g, const float* a_log,
                     const float* dt_bias, double lower_bound, float* out) {
  for (long i = 0; i < N; ++i)
    for (int h = 0; h < H; ++h)
      for (int c = 0; c < K; ++c) {
        long idx = (i * H + h) * K + c;
        out[idx] = to_f32(kda_o_decay(kda_o_bf16_to_double(raw_g[idx]), (double)a_log[h],
                                      (double)dt_bias[h * K + c], lower_bound));
      }
}

/* Plan steps of deferred RecoverSSM ([kernels page], the descriptions of
 * _defer_commit_kernel and _prepare_flush_plan_kernel), stated as a table:
 * every request is first given a class from its inputs, and each class then has
 * one fixed effect on the plan arrays. */
enum kda_o_plan_class {
  PLAN_UNTOUCHED, /* no state slot (padding, dummy rows) or no record slot */
  PLAN_DEFERRED,  /* its accepted tokens wait in its record slot */
  PLAN_COMMITTED  /* committed now by the caller (eager) */
};

static enum kda_o_plan_class plan_class(int slot, int record_row, int eager, int null_slot) {
  if (slot <= null_slot || record_row < 0) return PLAN_UNTOUCHED;
  return eager ? PLAN_COMMITTED : PLAN_DEFERRED;
}

/* Defer: a deferred request's commit length becomes the pending replay of its
 * record slot and no commit runs for it (its length becomes 0); a committed
 * one leaves nothing pending and keeps its plan; an untouched one changes no
 * pending count and no length. */
void kda_o_defer(int B, const int32_t* state_indices, int32_t* commit_lens,
                 const int32_t* record_rows, int32_t* pending, const int32_t* eager,
                 int null_slot) {
  enum kda_o_plan_class* cls = (enum kda_o_plan_class*)malloc(sizeof(*cls) * (size_t)(B > 0 ? B : 1));
  for (int b = 0; b < B; ++b)
    cls[b] = plan_class(state_indices[b], record_rows[b], eager ? eager[b] != 0 : 0, null_slot);
  for (int b = 0; b < B; ++b) {
    switch (cls[b]) {
      case PLAN_DEFERRED:
        pending[record_rows[b]] = commit_lens[b];
        commit_lens[b] = 0;
        break;
      case PLAN_COMMITTED:
        pending[record_rows[b]] = 0;
        break;
      case PLAN_UNTOUCHED:
        break;
    }
  }
  free(cls);
}

/* Flush plan: the commit that folds each request's pending replay into its
 * own checkpoint in place. Request b's entry: the commit reads and writes its
 * own slot (final index = its slot), stores no boundary (null slot, length
 * 0), and replays the pending count of its record slot, clamped to the window
 * [0, spec_query_len]; a request without a state slot, without a record slot
 * or with nothing pending replays nothing. The pending counts are read only. */
struct kda_o_flush_entry {
  int32_t len, final_slot, boundary, boundary_len;
};

void kda_o_flush_plan(int B, int spec_query_len, const int32_t* state_indices,
                      const int32_t* record_rows, const int32_t* pending, int32_t* commit_lens,
                      int32_t* final_indices, int32_t* boundaries, int32_t* boundary_lens,
                      int null_slot) {
  for (int b = 0; b < B; ++b) {
    const int slot = state_indices[b];
    const int waiting = record_rows[b] >= 0 ? pending[record_rows[b]] : 0;
    const int replay = waiting < 0 ? 0 : (waiting > spec_query_len ? spec_query_len : waiting);
    struct kda_o_flush_entry e;
    e.final_slot = slot;
    e.boundary = null_slot;
    e.boundary_len = 0;
    e.len = (slot > null_slot) ? replay : 0;
    commit_lens[b] = e.len;
    final_indices[b] = e.final_slot;
    boundaries[b] = e.boundary;
    boundary_lens[b] = e.boundary_len;
  }
}

/* Array forms of the two conversions (for the tests). */
void kda_o_round_bf16_buf(long n, const double* x, uint16_t* out) {
  for (long i = 0; i < n; ++i) out[i] = kda_o_double_to_bf16(x[i]);
}

void kda_o_bf16_to_double_buf(long n, const uint16_t* x, double* out) {
  for (long i = 0; i < n; ++i) out[i] = kda_o_bf16_to_double(x[i]);
}
