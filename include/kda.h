/*
 * kda.h — C ABI of the MI355X (gfx950) KDA gated delta-rule state-update library
 * (libkda.so): the bounded gate decay, the RecoverSSM commit, the stock verify,
 * the fused replay+verify (optionally with its convolution prologue), the
 * low-rank gate projection, and the two plan steps of deferred RecoverSSM.
 *
 * Sources are the vLLM API pages on Kimi-K3 KDA, cited by page title:
 *   [commit page]  vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.commit
 *   [kernels page] vllm.models.kimi_k3.nvidia.specialized_decode.recoverssm.kernels
 *   [fused page]   vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.fused
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Dimensions are fixed: K = V = 128 key and value channels per head. A head's
 *    state page is S[v][c] (row v = value channel, column c = key channel),
 *    128 x 128, contiguous; a slot holds H pages: state[slot][h][v][c].
 *  - Every pointer argument is a DEVICE pointer unless it says "host". Buffers
 *    are owned by the caller; the library allocates nothing, keeps no state
 *    of the computation between calls and never synchronises: work is
 *    enqueued on `stream` (a hipStream_t, NULL for the default stream) and
 *    the call returns.
 *  - BF16 tensors are passed as uint16_t bit patterns; index arrays are int32.
 *  - Return value: KDA_OK (0), KDA_EINVAL for a bad argument (nothing is
 *    launched), KDA_ELAUNCH when the HIP launch fails. kda_last_error() gives a
 *    message for the last failure on the calling thread.
 *  - Validation reads no device memory (the calls can be captured into a HIP
 *    graph). Device-side index data (slots, lengths, record rows, pending
 *    counts) is not range-checked: slots must lie in the pool, record rows in
 *    the record arrays. Requests of one call must not share a destination,
 *    boundary or record row, and no request's source may be another request's
 *    destination (their pages would race).
 *  - For that reason the pool's slot count and the record arrays' row count
 *    are not arguments: the kernels would only carry them, since the indices
 *    that must stay below them are device data that validation does not read.
 *    The caller sizes the pool and the records; a Python binding that sees
 *    the tensors can check them (spec_decode_amd checks the per-request arrays'
 *    lengths against batch).
 *  - Base pointers, strides and row pitches must keep every 16-byte vector
 *    access aligned; the library rejects them otherwise.
 *  - A slot index <= null_slot means "no state" (padding rows).
 *  - batch == 0 (or tokens == 0 for kda_decay) returns KDA_OK with no launch.
 *  - Launches whose state pages exceed the GPU's 256 MB memory-side cache
 *    (kda_commit: batch x heads x layers pages; kda_fused_replay_verify and
 *    kda_fused_conv_replay_verify on FP32 pools: batch x heads pages) write
 *    their pages with write-through, no-reuse stores, at two workgroups per
 *    CU (where a kernel's own LDS would allow more, extra dynamic LDS, sized
 *    on the first such launch of each kernel from its static LDS; this is the
 *    library's only retained host data). The results are bit-identical to
 *    those of smaller launches, except for kda_commit on FP32 pools: its
 *    streaming launches fold on the matrix cores (the products of up to four
 *    tokens summed in one instruction) where smaller ones add one token at a
 *    time, so the two can differ by FP32 rounding of the fold.
 */
#ifndef KDA_H
#define KDA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 7

#define KDA_OK 0
#define KDA_EINVAL 1
#define KDA_ELAUNCH 2

#define KDA_STATE_F32 0
#define KDA_STATE_BF16 1

#define KDA_HEAD_DIM 128
#define KDA_MAX_WINDOW 8

/* The message of the last failed call on this thread ("" after a success). */
const char* kda_last_error(void);

/* KDA_ABI_VERSION of the loaded library. */
int kda_abi_version(void);

/*
 * kda_decay — the bounded KDA gate decay, elementwise ([fused page],
 * KdaFused.decay):
 *     out[i][h][c] = exp(lower_bound * sigmoid(exp(a_log[h]) * (raw_g[i][h][c] + dt_bias[h][c])))
 *
 *   raw_g     BF16 [tokens][heads][128], contiguous
 *   a_log     FP32 [heads]
 *   dt_bias   FP32 [heads][128]
 *   out       FP32 [tokens][heads][128], contiguous; written
 * lower_bound must be finite. Computed in FP32 (hardware exp2-based exp).
 */
int kda_decay(const uint16_t* raw_g, int64_t tokens, int heads, const float* a_log,
              const float* dt_bias, float lower_bound, float* out, void* stream);

/*
 * kda_commit — the RecoverSSM commit ([commit page], module docstring, KdaCommit
 * class docstring and kernel): for every (layer l, request b, head h) item with
 * n = commit_lens[b] > 0, sources[b] > null_slot, destinations[b] > null_slot and
 * a record row r >= 0 (r = record_rows[b], or b when record_rows is NULL):
 *
 *     S_n = S_0 diag(D_n) + sum_{t<n} u_t (kn_t * P_t)^T,
 *     D_n = prod_{s<n} d_s,   P_t = prod_{t<s<n} d_s,
 *
 * with S_0 the source page, u_t the recorded corrections, kn_t the recorded raw
 * keys L2-normalised (eps 1e-6 inside the root), d_t the decays of the recorded
 * raw gates under a_log[l][h], dt_bias[l][h][:]. S_n is written to the
 * destination page (which may equal the source: an in-place commit). n is
 * capped at `window`. When boundaries and boundary_lens are given (align) and
 * m = boundary_lens[b] > 0 with boundaries[b] > null_slot, S_m (m capped at n)
 * is also written to the boundary page. Items that are not live write nothing.
 * Arithmetic is FP32; stores round to the state dtype (BF16: nearest-even).
 *
 *   layers, heads        L >= 1 and H >= 1
 *   window               Q in 1..8: the records' token capacity and the cap on n
 *   batch                B requests
 *   state_dtype          KDA_STATE_F32 or KDA_STATE_BF16
 *   state_addrs          HOST array [L] of device base addresses of each layer's
 *                        state pool [slots][H][128][128]
 *   state_slot_strides   HOST array [L]: elements between slots (>= H*128*128)
 *   corr_addrs           HOST array [L]: FP32 corrections [rows][H][Q][128]
 *   corr_row_strides     HOST array [L]: elements between record rows (>= H*Q*128)
 *   kg_addrs             HOST array [L]: BF16 key/gate records [rows][H][Q][256]
 *                        (raw key in 0..127, raw gate in 128..255)
 *   kg_row_strides       HOST array [L]: elements between record rows (>= H*Q*256)
 *   a_log                FP32 [L][H];  dt_bias  FP32 [L][H][128]
 *   sources, commit_lens, destinations      int32 [B]
 *   boundaries, boundary_lens               int32 [B], or both NULL (align off)
 *   record_rows          int32 [B] or NULL (row b)
 *   lower_bound          finite;  null_slot  the padding slot id (usually 0)
 * Any number of layers is accepted (the library launches them in chunks).
 */
int kda_commit(int layers, int heads, int window, int batch, int state_dtype,
               const uint64_t* state_addrs, const int64_t* state_slot_strides,
               const uint64_t* corr_addrs, const int64_t* corr_row_strides,
               const uint64_t* kg_addrs, const int64_t* kg_row_strides,
               const float* a_log, const float* dt_bias, const int32_t* sources,
               const int32_t* commit_lens, const int32_t* destinations,
               const int32_t* boundaries, const int32_t* boundary_lens,
               const int32_t* record_rows, float lower_bound, int null_slot, void* stream);

/*
 * kda_verify — the stock RecoverSSM verify of a window of `tokens` new tokens
 * per request, which never writes the checkpoint ([kernels page],
 * kda_recoverssm_verify; the recurrence of the [fused page] module docstring).
 * For every (request b, head h) with slot = state_indices[b]:
 *  - slot <= null_slot: out rows of the item are zero; nothing else is written;
 *  - otherwise, from S = state page (FP32, or BF16 widened exactly), for t < tokens:
 *        S <- S diag(d_t);  u_t = beta_t (v_t - S kn_t);  S <- S + u_t kn_t^T;  o_t = S q_t
 *    computed in the chunked (WY) form from the unmodified page; o_t -> out
 *    (BF16); with beta_t = sigmoid(raw_beta), kn_t the L2-normalised key, q_t
 *    used as given;
 *  - record row r = record_rows[b] (or b when NULL); r >= 0: corrections
 *    [r][h][t][:] = u_t (FP32), key/gate [r][h][t][0:128] = k_t bits and
 *    [128:256] = raw gate bits, for t < tokens (later record tokens untouched).
 *
 *   heads, tokens (1..8), batch
 *   q, k, raw_g          BF16 [batch*tokens][heads][128], contiguous
 *   v                    BF16 [batch*tokens][heads][128], contiguous
 *   raw_beta             BF16 [batch*tokens][heads]
 *   a_log                FP32 [heads];  dt_bias  FP32 [heads][128]
 *   state_dtype          KDA_STATE_F32 or KDA_STATE_BF16: the element type of state
 *   state                pool [slots][heads][128][128] of state_dtype (BF16 as bits);
 *                        read only
 *   state_slot_stride    elements between slots (>= heads*128*128; slots 16-byte
 *                        aligned: a multiple of 4 for FP32, of 8 for BF16)
 *   state_indices        int32 [batch]
 *   corr                 FP32 records [rows][heads][record_tokens][128]
 *   kg                   BF16 records [rows][heads][record_tokens][256]
 *   record_tokens        RQ in tokens..8
 *   record_rows          int32 [batch] or NULL
 *   query_start_loc      int32 [batch + 1] or NULL (variable-length windows,
 *                        [kernels page] kda_recoverssm_verify's query metadata):
 *                        request b's tokens are the rows qsl[b] .. qsl[b] + L - 1
 *                        of q, k, v, raw_g, raw_beta, gate and out, with
 *                        L = clamp(qsl[b+1] - qsl[b], 0, tokens). L = 0 is padding:
 *                        nothing is read or written for the item. Records are
 *                        rewritten for t < L; later record tokens keep their
 *                        values. NULL: L = tokens and rows b*tokens + t
 *   gate, norm_weight    the optional gated RMSNorm output stage ([fused page],
 *                        KdaFused output stage), both NULL to write o itself:
 *                        gate BF16 [batch*tokens][heads*128], norm_weight FP32 [128]
 *                        (shared by the heads). Per (token, head), with o_bf = BF16(o),
 *                        out = BF16(o_bf * rsqrt(mean_v(o_bf^2) + norm_eps)
 *                                   * norm_weight[v] * sigmoid(gate[v]))
 *   norm_eps             finite, >= 0 (used with gate)
 *   out                  BF16 [batch*tokens][heads*128]; written
 */
int kda_verify(int heads, int tokens, int batch, const uint16_t* q, const uint16_t* k,
               const uint16_t* v, const uint16_t* raw_g, const uint16_t* raw_beta,
               const float* a_log, const float* dt_bias, float lower_bound, int state_dtype,
               const void* state, int64_t state_slot_stride, const int32_t* state_indices,
               int null_slot, float* corr, uint16_t* kg, int record_tokens,
               const int32_t* record_rows, const int32_t* query_start_loc,
               const uint16_t* gate, const float* norm_weight, float norm_eps, uint16_t* out,
               void* stream);

/*
 * kda_fused_replay_verify — deferred RecoverSSM: the previous step's commit and
 * this step's verify in one pass over the state ([fused page], module
 * docstring and KdaFused). Arguments as kda_verify, plus `pending`; state is
 * read and written. For every (request b, head h) with slot > null_slot:
 *  1. r = record_rows[b]; n = clamp(pending[r], 0, record_tokens) if r >= 0,
 *     else 0; the n recorded tokens of row r are replayed onto the page in the
 *     commit's closed form (FP32 arithmetic) and S_n is written back to the same
 *     page when n > 0 (a BF16 pool stores S_n rounded to nearest even);
 *  2. the window is verified from S_n (the FP32 value, before any rounding to
 *     the pool's type) exactly as kda_verify does;
 *  3. r >= 0: the records of row r are rewritten for t < tokens, after every
 *     old record of the item was read.
 * pending is read only (the defer step of the next step rewrites it). Each
 * state byte is read once and written at most once.
 *
 *   record_rows          int32 [batch], required (< 0: no record row)
 *   pending              int32 [rows], indexed by record row
 *   query_start_loc      as kda_verify (an item with L = 0 does not replay)
 *   boundaries,          int32 [batch] each, both or neither (align, as kda_commit's):
 *   boundary_lens        for an item whose replay runs (n > 0), with bnd =
 *                        boundaries[b] > null_slot and m = boundary_lens[b] > 0,
 *                        S_min(m, n) is also stored to slot bnd (same page
 *                        layout and dtype); the fold then runs in two stages,
 *                        tokens [0, min(m, n)) and the rest. Boundary slots must
 *                        not be any request's slot or another's boundary.
 *   gate, norm_weight, norm_eps   the optional output stage, as kda_verify
 */
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
                            void* stream);

/*
 * kda_fused_conv_replay_verify — kda_fused_replay_verify with its convolution
 * prologue ([fused page], KdaFused: the convolution, its SiLU and the q/k
 * normalisation): q, k and v are computed from pre-activations instead of
 * being passed. For every (request b, head h) with slot > null_slot, part p
 * (0 q, 1 k, 2 v) and head channel c, with column j = p*heads*128 + h*128 + c:
 *  - the window w[i] = conv_state[slot*conv_slot_stride + j*conv_channel_stride
 *    + i*conv_tap_stride], i < record_tokens + 2, holds the previous step's
 *    [2 history values, its inputs]; the 3 taps are w[o..o+2] with
 *    o = max(n - 1, 0), n the item's replay count (step 1 of the fused step);
 *  - seq = [taps, x[b*tokens + t][j] for t < tokens];
 *    pre_t = conv_bias[j] + sum_{i<4} conv_weight[p][i][h*128 + c] * seq[t + i]
 *    (0 for a NULL bias; weight 3 meets the current input), and the part's
 *    output is y_t = BF16(SiLU(pre_t)), SiLU(a) = a / (1 + exp(-a));
 *    this rounding is decided in FP32 by fixed steps: an fma chain in tap order
 *    from the bias, exp by Cody-Waite reduction (ln 2 split at 16 fraction
 *    bits) and the degree-7 Taylor polynomial in Horner form on [-80, 80], an
 *    IEEE divide, round to nearest even;
 *  - q_t = y_q * (sum_c y_q^2 + 1e-6)^-1/2 * q_scale; k_t = y_k (normalised at
 *    use, as always; the record keeps y_k's bits); v_t = y_v;
 *  - the window is rewritten as [tap 1, tap 2, x_0 .. x_{tokens-1}]; entries
 *    past tokens + 1 keep their values.
 * The rest is kda_fused_replay_verify with fixed windows (rows b*tokens + t; no
 * query_start_loc). Null-slot items write only their zero outputs.
 *
 *   x                    BF16 [batch*tokens] rows of x_row_stride elements
 *                        (>= 3*heads*128): the q | k | v pre-activations in
 *                        columns [0, 3*heads*128); other columns are not read
 *   conv_weight          BF16 [3][4][heads*128]
 *   conv_bias            BF16 [3*heads*128], or NULL for none
 *   conv_state           BF16 window pool, read and written; strides >= 1 in
 *                        elements. Windows of distinct (slot, column) pairs
 *                        must not overlap. Dim-first [slots][3*heads*128][W]:
 *                        strides (3*heads*128*W, W, 1); window-major
 *                        [slots][W][3*heads*128]: (3*heads*128*W, 1, 3*heads*128);
 *                        W >= record_tokens + 2. A dim-first pool with
 *                        W = record_tokens + 2 (tap stride 1, channel stride W),
 *                        a slot stride that is a multiple of 8 and a 16-byte
 *                        aligned base is moved in 16-byte chunks, each wave's
 *                        64 windows as one block. A window-major pool (channel
 *                        stride 1) whose tap and slot strides are multiples
 *                        of 8 and whose base is 16-byte aligned, with x 16-byte
 *                        aligned and x_row_stride a multiple of 8, moves its
 *                        taps, inputs and new entries in 16-byte chunks through
 *                        a per-wave LDS stage. Other pools use 2-byte accesses
 *                        (the results are the same bits)
 *   q_scale              finite (the pages use 128^-1/2)
 *   raw_g, raw_beta, a_log, dt_bias, lower_bound, state_dtype, state,
 *   state_slot_stride, state_indices, null_slot, corr, kg, record_tokens,
 *   record_rows, pending, boundaries, boundary_lens, gate, norm_weight, norm_eps,
 *   out                  as kda_fused_replay_verify
 */
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
                                 void* stream);

/*
 * kda_gate_projection — the low-rank gate projection that produces raw_g
 * ([fused page], KdaFused: the gate projection):
 *     raw_g[t][f] = BF16(sum_{j<128} f_a[t][j] * f_b[f][j]),  f < heads*128,
 * FP32 accumulation (BF16 matrix cores), rounded to nearest even. The result
 * is the raw_g operand of kda_verify / kda_fused_replay_verify /
 * kda_fused_conv_replay_verify and of the records. The FP32 sum's order is the
 * hardware's: where the exact sum lies within FP32 rounding of a BF16 rounding
 * boundary, the result can be the neighbouring BF16 value.
 *
 *   tokens               >= 0 (0: no launch)
 *   heads                1..65535
 *   f_a                  BF16 [tokens] rows of f_a_row_stride elements (>= 128,
 *                        a multiple of 8); columns 0..127 are read (e.g. a column
 *                        slice of a packed projection row)
 *   f_b                  BF16 [heads*128][128], row-major
 *   raw_g                BF16 [tokens][heads][128]; written
 * All three 16-byte aligned.
 */
int kda_gate_projection(int64_t tokens, int heads, const uint16_t* f_a,
                        int64_t f_a_row_stride, const uint16_t* f_b, uint16_t* raw_g,
                        void* stream);

/*
 * kda_defer_commit — the defer step of deferred RecoverSSM ([kernels page],
 * _defer_commit_kernel). For each request b with record_rows[b] >= 0 and
 * state_indices[b] > null_slot: if eager != NULL and eager[b] != 0,
 * pending[record_rows[b]] = 0 and commit_lens[b] is kept; otherwise
 * pending[record_rows[b]] = commit_lens[b] and commit_lens[b] = 0. Other
 * requests change nothing.
 *   state_indices, record_rows, eager (or NULL)   int32 [batch]
 *   commit_lens          int32 [batch], read and written
 *   pending              int32 [rows], written
 */
int kda_defer_commit(int batch, const int32_t* state_indices, int32_t* commit_lens,
                     const int32_t* record_rows, int32_t* pending, const int32_t* eager,
                     int null_slot, void* stream);

/*
 * kda_flush_plan — the plan of an in-place commit of every pending replay
 * ([kernels page], _prepare_flush_plan_kernel). For each request b:
 *   n = record_rows[b] >= 0 ? pending[record_rows[b]] : 0, clamped to
 *   [0, spec_query_len]; commit_lens[b] = (state_indices[b] > null_slot && n > 0) ? n : 0;
 *   final_indices[b] = state_indices[b]; boundaries[b] = null_slot; boundary_lens[b] = 0.
 * pending is read only.
 *   spec_query_len       1..8
 *   state_indices, record_rows   int32 [batch]
 *   pending              int32 [rows]
 *   commit_lens, final_indices, boundaries, boundary_lens   int32 [batch], written
 */
int kda_flush_plan(int batch, int spec_query_len, const int32_t* state_indices,
                   const int32_t* record_rows, const int32_t* pending, int32_t* commit_lens,
                   int32_t* final_indices, int32_t* boundaries, int32_t* boundary_lens,
                   int null_slot, void* stream);

/*
 * kda_page_rw_probe — measurement aid, not a step of the method: loads every
 * page of every named slot (state_indices[b] > null_slot, all heads) and stores
 * it back unchanged, in the access pattern of the fused kernel over FP32 pools
 * larger than the memory-side cache (contiguous 1 KiB pieces per wave load
 * with the no-reuse hint, an LDS transpose to 16x16 tiles, one write-through
 * 16-byte store per lane and tile, one workgroup per page). Its rate
 * is the in-place read+write ceiling of the pool on the running GPU; the
 * benchmark reports its kernels against it next to the HBM peak. The pool's
 * contents are unchanged. Arguments as kda_fused_replay_verify's state,
 * state_slot_stride, state_indices and null_slot.
 */
int kda_page_rw_probe(int heads, int batch, float* state, int64_t state_slot_stride,
                      const int32_t* state_indices, int null_slot, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
