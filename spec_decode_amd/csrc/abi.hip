// The extern "C" boundary of libkda: argument checks (host values only, no
// device reads), then one launch on the caller's stream. Semantics and argument
// layouts are documented in include/kda.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/kda.h"
#include "kda_device.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return KDA_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(KDA_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define KDA_REQUIRE(cond, ...) \
  do {                         \
    if (!(cond)) return fail(KDA_EINVAL, __VA_ARGS__); \
  } while (0)

constexpr int64_t kPage = (int64_t)kda::K * kda::V;

// The convolution prologue's operands (kda_fused_conv_replay_verify).
struct ConvArgs {
  const uint16_t* x;
  int64_t x_row_stride;
  const uint16_t* weight;
  const uint16_t* bias;
  uint16_t* state;
  int64_t slot_stride, channel_stride, tap_stride;
  float q_scale;
};

}  // namespace

extern "C" {

const char* kda_last_error(void) { return g_last_error.c_str(); }

int kda_abi_version(void) { return KDA_ABI_VERSION; }

int kda_decay(const uint16_t* raw_g, int64_t tokens, int heads, const float* a_log,
              const float* dt_bias, float lower_bound, float* out, void* stream) {
  KDA_REQUIRE(tokens >= 0, "kda_decay: tokens must be >= 0 (got %lld)", (long long)tokens);
  KDA_REQUIRE(heads >= 1, "kda_decay: heads must be >= 1 (got %d)", heads);
  KDA_REQUIRE(std::isfinite(lower_bound), "kda_decay: lower_bound must be finite");
  if (tokens == 0) return ok();
  KDA_REQUIRE(raw_g && a_log && dt_bias && out, "kda_decay: null pointer argument");
  KDA_REQUIRE(aligned16(raw_g) && aligned16(out) && aligned16(dt_bias),
              "kda_decay: raw_g, dt_bias and out must be 16-byte aligned");
  // The kernel strides over 4-channel chunks with a capped grid; the only
  // limit is the element count's 64-bit range.
  KDA_REQUIRE(tokens <= INT64_MAX / kda::K / heads, "kda_decay: tensor too large");
  return launched(kda::launch_decay(raw_g, tokens, heads, a_log, dt_bias, lower_bound, out,
                                    reinterpret_cast<hipStream_t>(stream)),
                  "kda_decay");
}

int kda_commit(int layers, int heads, int window, int batch, int state_dtype,
               const uint64_t* state_addrs, const int64_t* state_slot_strides,
               const uint64_t* corr_addrs, const int64_t* corr_row_strides,
               const uint64_t* kg_addrs, const int64_t* kg_row_strides, const float* a_log,
               const float* dt_bias, const int32_t* sources, const int32_t* commit_lens,
               const int32_t* destinations, const int32_t* boundaries,
               const int32_t* boundary_lens, const int32_t* record_rows, float lower_bound,
               int null_slot, void* stream) {
  KDA_REQUIRE(layers >= 1, "kda_commit: layers must be >= 1 (got %d)", layers);
  KDA_REQUIRE(heads >= 1 && heads <= 65535, "kda_commit: heads must be in 1..65535 (got %d)",
              heads);
  KDA_REQUIRE(window >= 1 && window <= KDA_MAX_WINDOW,
              "kda_commit: window must be in 1..8 (got %d)", window);
  KDA_REQUIRE(batch >= 0 && batch <= 65535, "kda_commit: batch must be in 0..65535 (got %d)",
              batch);
  KDA_REQUIRE(state_dtype == KDA_STATE_F32 || state_dtype == KDA_STATE_BF16,
              "kda_commit: state_dtype must be KDA_STATE_F32 or KDA_STATE_BF16");
  KDA_REQUIRE(std::isfinite(lower_bound), "kda_commit: lower_bound must be finite");
  KDA_REQUIRE((boundaries == nullptr) == (boundary_lens == nullptr),
              "kda_commit: boundaries and boundary_lens must be given together");
  if (batch == 0) return ok();
  KDA_REQUIRE(state_addrs && state_slot_strides && corr_addrs && corr_row_strides && kg_addrs &&
                  kg_row_strides,
              "kda_commit: null address or stride table");
  KDA_REQUIRE(a_log && dt_bias && sources && commit_lens && destinations,
              "kda_commit: null pointer argument");
  const bool bf16 = state_dtype == KDA_STATE_BF16;
  const int64_t es = bf16 ? 2 : 4;
  for (int l = 0; l < layers; ++l) {
    KDA_REQUIRE(state_addrs[l] && corr_addrs[l] && kg_addrs[l],
                "kda_commit: layer %d has a null base address", l);
    KDA_REQUIRE((state_addrs[l] & 15u) == 0 && (corr_addrs[l] & 15u) == 0 &&
                    (kg_addrs[l] & 15u) == 0,
                "kda_commit: layer %d base addresses must be 16-byte aligned", l);
    KDA_REQUIRE(state_slot_strides[l] >= heads * kPage && (state_slot_strides[l] * es) % 16 == 0,
                "kda_commit: layer %d slot stride %lld must be >= heads*128*128 and keep "
                "slots 16-byte aligned",
                l, (long long)state_slot_strides[l]);
    KDA_REQUIRE(corr_row_strides[l] >= (int64_t)heads * window * kda::V &&
                    (corr_row_strides[l] * 4) % 16 == 0,
                "kda_commit: layer %d correction row stride %lld must be >= heads*window*128 "
                "and a multiple of 4",
                l, (long long)corr_row_strides[l]);
    KDA_REQUIRE(kg_row_strides[l] >= (int64_t)heads * window * 2 * kda::K &&
                    (kg_row_strides[l] * 2) % 16 == 0,
                "kda_commit: layer %d key/gate row stride %lld must be >= heads*window*256 and "
                "a multiple of 8",
                l, (long long)kg_row_strides[l]);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int l0 = 0; l0 < layers; l0 += kda::COMMIT_LAYERS_PER_LAUNCH) {
    const int nl = layers - l0 < kda::COMMIT_LAYERS_PER_LAUNCH ? layers - l0
                                                               : kda::COMMIT_LAYERS_PER_LAUNCH;
    kda::CommitParams p{};
    for (int i = 0; i < nl; ++i) {
      p.layer[i].state = reinterpret_cast<void*>(state_addrs[l0 + i]);
      p.layer[i].corr = reinterpret_cast<const float*>(corr_addrs[l0 + i]);
      p.layer[i].kg = reinterpret_cast<const uint16_t*>(kg_addrs[l0 + i]);
      p.layer[i].state_stride = state_slot_strides[l0 + i];
      p.layer[i].corr_stride = corr_row_strides[l0 + i];
      p.layer[i].kg_stride = kg_row_strides[l0 + i];
    }
    p.a_log = a_log + (int64_t)l0 * heads;
    p.dt_bias = dt_bias + (int64_t)l0 * heads * kda::K;
    p.sources = sources;
    p.lens = commit_lens;
    p.dests = destinations;
    p.bounds = boundaries;
    p.blens = boundary_lens;
    p.rows = record_rows;
    p.heads = heads;
    p.null_slot = null_slot;
    p.lb = lower_bound;
    const int rc = launched(
        kda::launch_commit(p, window, bf16, boundaries != nullptr, batch, nl, s), "kda_commit");
    if (rc != KDA_OK) return rc;
  }
  return ok();
}

static int verify_common(const char* who, bool fused, int heads, int tokens, int batch,
                         const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* raw_g, const uint16_t* raw_beta, const float* a_log,
                         const float* dt_bias, float lower_bound, int state_dtype,
                         void* state, int64_t state_slot_stride, const int32_t* state_indices,
                         int null_slot, float* corr, uint16_t* kg, int record_tokens,
                         const int32_t* record_rows, const int32_t* pending,
                         const int32_t* query_start_loc, const int32_t* boundaries,
                         const int32_t* boundary_lens, const uint16_t* gate,
                         const float* norm_weight, float norm_eps, uint16_t* out,
                         void* stream, const ConvArgs* conv = nullptr) {
  KDA_REQUIRE(heads >= 1 && heads <= 65535, "%s: heads must be in 1..65535 (got %d)", who,
              heads);
  KDA_REQUIRE(tokens >= 1 && tokens <= KDA_MAX_WINDOW, "%s: tokens must be in 1..8 (got %d)",
              who, tokens);
  KDA_REQUIRE(batch >= 0 && batch <= 65535, "%s: batch must be in 0..65535 (got %d)", who,
              batch);
  KDA_REQUIRE(record_tokens >= tokens && record_tokens <= KDA_MAX_WINDOW,
              "%s: record_tokens must be in tokens..8 (got %d with tokens %d)", who,
              record_tokens, tokens);
  KDA_REQUIRE(std::isfinite(lower_bound), "%s: lower_bound must be finite", who);
  KDA_REQUIRE(state_dtype == KDA_STATE_F32 || state_dtype == KDA_STATE_BF16,
              "%s: state_dtype must be KDA_STATE_F32 or KDA_STATE_BF16", who);
  KDA_REQUIRE((gate == nullptr) == (norm_weight == nullptr),
              "%s: gate and norm_weight must be given together", who);
  KDA_REQUIRE((boundaries == nullptr) == (boundary_lens == nullptr),
              "%s: boundaries and boundary_lens must be given together", who);
  KDA_REQUIRE(gate == nullptr || (std::isfinite(norm_eps) && norm_eps >= 0.f),
              "%s: norm_eps must be finite and >= 0", who);
  if (conv != nullptr) {
    KDA_REQUIRE(std::isfinite(conv->q_scale), "%s: q_scale must be finite", who);
    KDA_REQUIRE(conv->x_row_stride >= 3 * (int64_t)heads * kda::K,
                "%s: x_row_stride %lld must be >= 3*heads*128", who,
                (long long)conv->x_row_stride);
    KDA_REQUIRE(conv->slot_stride >= 1 && conv->channel_stride >= 1 && conv->tap_stride >= 1,
                "%s: convolution window strides must be >= 1", who);
  }
  if (batch == 0) return ok();
  if (conv != nullptr) {
    KDA_REQUIRE(conv->x && conv->weight && conv->state, "%s: null pointer argument", who);
  } else {
    KDA_REQUIRE(q && k && v, "%s: null pointer argument", who);
  }
  KDA_REQUIRE(raw_g && raw_beta && a_log && dt_bias && state && state_indices && corr && kg &&
                  out,
              "%s: null pointer argument", who);
  if (fused)
    KDA_REQUIRE(record_rows && pending, "%s: record_rows and pending are required", who);
  KDA_REQUIRE(aligned16(state) && aligned16(out),
              "%s: state and out must be 16-byte aligned", who);
  const bool bf16 = state_dtype == KDA_STATE_BF16;
  const int64_t es = bf16 ? 2 : 4;
  KDA_REQUIRE(state_slot_stride >= heads * kPage && (state_slot_stride * es) % 16 == 0,
              "%s: state_slot_stride %lld must be >= heads*128*128 and keep slots 16-byte "
              "aligned",
              who, (long long)state_slot_stride);
  kda::VerifyParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = raw_g;
  p.rb = raw_beta;
  p.a_log = a_log;
  p.dt_bias = dt_bias;
  p.state = state;
  p.slot_stride = state_slot_stride;
  p.slots = state_indices;
  p.rows = record_rows;
  p.pending = pending;
  p.qsl = query_start_loc;
  p.bounds = boundaries;
  p.blens = boundary_lens;
  p.corr = corr;
  p.kg = kg;
  p.out = out;
  p.gate = gate;
  p.norm_w = norm_weight;
  p.norm_eps = norm_eps;
  p.rq = record_tokens;
  p.heads = heads;
  p.null_slot = null_slot;
  p.lb = lower_bound;
  if (conv != nullptr) {
    p.x = conv->x;
    p.x_stride = conv->x_row_stride;
    p.conv_w = conv->weight;
    p.conv_b = conv->bias;
    p.conv = conv->state;
    p.conv_ss = conv->slot_stride;
    p.conv_cs = conv->channel_stride;
    p.conv_ts = conv->tap_stride;
    p.q_scale = conv->q_scale;
  }
  return launched(
      kda::launch_verify(p, tokens, fused, bf16, batch, reinterpret_cast<hipStream_t>(stream)),
      who);
}

int kda_verify(int heads, int tokens, int batch, const uint16_t* q, const uint16_t* k,
               const uint16_t* v, const uint16_t* raw_g, const uint16_t* raw_beta,
               const float* a_log, const float* dt_bias, float lower_bound, int state_dtype,
               const void* state, int64_t state_slot_stride, const int32_t* state_indices,
               int null_slot, float* corr, uint16_t* kg, int record_tokens,
               const int32_t* record_rows, const int32_t* query_start_loc,
               const uint16_t* gate, const float* norm_weight, float norm_eps, uint16_t* out,
               void* stream) {
  return verify_common("kda_verify", false, heads, tokens, batch, q, k, v, raw_g, raw_beta,
                       a_log, dt_bias, lower_bound, state_dtype, const_cast<void*>(state),
                       state_slot_stride, state_indices, null_slot, corr, kg, record_tokens,
                       record_rows, nullptr, query_start_loc, nullptr, nullptr, gate,
                       norm_weight, norm_eps, out, stream);
}

int kda_fused_replay_verify(int heads, int tokens, int batch, const uint16_t* q,
                            const uint16_t* k, const uint16_t* v, const uint16_t* raw_g,
                            const uint16_t* raw_beta, const float* a_log, const float* dt_bias,
                            float lower_bound, int state_dtype, void* state,
                            int64_t state_slot_stride, const int32_t* state_indices,
                            int null_slot, float* corr, uint16_t* kg, int record_tokens,
                            const int32_t* record_rows, const int32_t* pending,
                            const int32_t* query_start_loc, const int32_t* boundaries,
                            const int32_t* boundary_lens, const uint16_t* gate,
                            const float* norm_weight, float norm_eps, uint16_t* out,
                            void* stream) {
  return verify_common("kda_fused_replay_verify", true, heads, tokens, batch, q, k, v, raw_g,
                       raw_beta, a_log, dt_bias, lower_bound, state_dtype, state,
                       state_slot_stride, state_indices, null_slot, corr, kg, record_tokens,
                       record_rows, pending, query_start_loc, boundaries, boundary_lens, gate,
                       norm_weight, norm_eps, out, stream);
}

int kda_fused_conv_replay_verify(int heads, int tokens, int batch, const uint16_t* x,
                                 int64_t x_row_stride, const uint16_t* conv_weight,
                                 const uint16_t* conv_bias, uint16_t* conv_state,
                                 int64_t conv_slot_stride, int64_t conv_channel_stride,
                                 int64_t conv_tap_stride, float q_scale, const uint16_t* raw_g,
                                 const uint16_t* raw_beta, const float* a_log,
                                 const float* dt_bias, float lower_bound, int state_dtype,
                                 void* state, int64_t state_slot_stride,
                                 const int32_t* state_indices, int null_slot, float* corr,
                                 uint16_t* kg, int record_tokens, const int32_t* record_rows,
                                 const int32_t* pending, const int32_t* boundaries,
                                 const int32_t* boundary_lens, const uint16_t* gate,
                                 const float* norm_weight, float norm_eps, uint16_t* out,
                                 void* stream) {
  const ConvArgs conv{x,          x_row_stride,     conv_weight,         conv_bias, conv_state,
                      conv_slot_stride, conv_channel_stride, conv_tap_stride, q_scale};
  return verify_common("kda_fused_conv_replay_verify", true, heads, tokens, batch, nullptr,
                       nullptr, nullptr, raw_g, raw_beta, a_log, dt_bias, lower_bound,
                       state_dtype, state, state_slot_stride, state_indices, null_slot, corr, kg,
                       record_tokens, record_rows, pending, nullptr, boundaries, boundary_lens,
                       gate, norm_weight, norm_eps, out, stream, &conv);
}

int kda_gate_projection(int64_t tokens, int heads, const uint16_t* f_a,
                        int64_t f_a_row_stride, const uint16_t* f_b, uint16_t* raw_g,
                        void* stream) {
  KDA_REQUIRE(tokens >= 0, "kda_gate_projection: tokens must be >= 0 (got %lld)",
              (long long)tokens);
  KDA_REQUIRE(heads >= 1 && heads <= 65535,
              "kda_gate_projection: heads must be in 1..65535 (got %d)", heads);
  KDA_REQUIRE(f_a_row_stride >= kda::K && f_a_row_stride % 8 == 0,
              "kda_gate_projection: f_a_row_stride %lld must be >= 128 and a multiple of 8",
              (long long)f_a_row_stride);
  KDA_REQUIRE((tokens + 63) / 64 < ((int64_t)1 << 31), "kda_gate_projection: too many tokens");
  if (tokens == 0) return ok();
  KDA_REQUIRE(f_a && f_b && raw_g, "kda_gate_projection: null pointer argument");
  KDA_REQUIRE(aligned16(f_a) && aligned16(f_b) && aligned16(raw_g),
              "kda_gate_projection: f_a, f_b and raw_g must be 16-byte aligned");
  return launched(kda::launch_gate_projection(f_a, f_a_row_stride, f_b, raw_g, tokens, heads,
                                              reinterpret_cast<hipStream_t>(stream)),
                  "kda_gate_projection");
}

int kda_defer_commit(int batch, const int32_t* state_indices, int32_t* commit_lens,
                     const int32_t* record_rows, int32_t* pending, const int32_t* eager,
                     int null_slot, void* stream) {
  KDA_REQUIRE(batch >= 0, "kda_defer_commit: batch must be >= 0 (got %d)", batch);
  if (batch == 0) return ok();
  KDA_REQUIRE(state_indices && commit_lens && record_rows && pending,
              "kda_defer_commit: null pointer argument");
  return launched(kda::launch_defer(batch, state_indices, commit_lens, record_rows, pending,
                                    eager, null_slot, reinterpret_cast<hipStream_t>(stream)),
                  "kda_defer_commit");
}

int kda_flush_plan(int batch, int spec_query_len, const int32_t* state_indices,
                   const int32_t* record_rows, const int32_t* pending, int32_t* commit_lens,
                   int32_t* final_indices, int32_t* boundaries, int32_t* boundary_lens,
                   int null_slot, void* stream) {
  KDA_REQUIRE(batch >= 0, "kda_flush_plan: batch must be >= 0 (got %d)", batch);
  KDA_REQUIRE(spec_query_len >= 1 && spec_query_len <= KDA_MAX_WINDOW,
              "kda_flush_plan: spec_query_len must be in 1..8 (got %d)", spec_query_len);
  if (batch == 0) return ok();
  KDA_REQUIRE(state_indices && record_rows && pending && commit_lens && final_indices &&
                  boundaries && boundary_lens,
              "kda_flush_plan: null pointer argument");
  return launched(kda::launch_flush_plan(batch, spec_query_len, state_indices, record_rows,
                                         pending, commit_lens, final_indices, boundaries,
                                         boundary_lens, null_slot,
                                         reinterpret_cast<hipStream_t>(stream)),
                  "kda_flush_plan");
}

int kda_page_rw_probe(int heads, int batch, float* state, int64_t state_slot_stride,
                      const int32_t* state_indices, int null_slot, void* stream) {
  KDA_REQUIRE(heads >= 1 && heads <= 65535, "kda_page_rw_probe: heads must be in 1..65535");
  KDA_REQUIRE(batch >= 0 && batch <= 65535, "kda_page_rw_probe: batch must be in 0..65535");
  if (batch == 0) return ok();
  KDA_REQUIRE(state && state_indices, "kda_page_rw_probe: null pointer argument");
  KDA_REQUIRE(aligned16(state), "kda_page_rw_probe: state must be 16-byte aligned");
  KDA_REQUIRE(state_slot_stride >= heads * kPage && state_slot_stride % 4 == 0,
              "kda_page_rw_probe: state_slot_stride must be >= heads*128*128 and a multiple of 4");
  return launched(kda::launch_page_rw(state, state_slot_stride, state_indices, batch, heads,
                                      null_slot, reinterpret_cast<hipStream_t>(stream)),
                  "kda_page_rw_probe");
}

}  // extern "C"
