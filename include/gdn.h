/*
 * gdn.h -- C ABI of the Gated DeltaNet (GDN) hot path for AMD Instinct MI355X
 * (gfx950).
 *
 * The method (sources are web pages; each entry point names the passage that
 * defines it):
 *   gate        g = softplus(alpha + dt_bias) * ssm_a, softplus(x) = x when
 *               x > 20 and log1p(exp(x)) otherwise; ssm_a = -exp(A_log) < 0
 *               (Winery-Strata, src/kernels/elementwise_parity.cpp, the
 *               gdn_gate block and its softplus-branch / negative-ssm_a notes).
 *   recurrence  per v-head, state S[Dv][Dk] in fp32 (rows index v, columns k):
 *               S *= exp(g); v' = beta * (v - S k); S += v' (outer) k;
 *               o = S (q * scale), the output read from the updated state
 *               (vllm.cpp, tests/vt/test_ops_gdn.cpp, "gdn decode:
 *               hand-computed single step" and the 3-token prefill table).
 *   q/k norm    x / sqrt(sum_d x_d^2 + eps), per (token, q/k head), q scaled
 *               after normalising (same file, the l2norm cases and
 *               PackedDecodeReference).
 *   GQA         v-head hv reads q/k head hv / (Hv / Hk) (same file, "GQA
 *               ratio 3 broadcast").
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except
 *     the return value of gdn_last_error().  The library allocates no device
 *     memory, frees nothing and never synchronises: each call enqueues its
 *     kernels on `stream` and returns; results are visible after the stream
 *     completes.  No call reads device data on the host, so calls can be
 *     captured into a HIP graph -- except with GDN_CHECK_SLOTS, which copies
 *     the slot table (and cu_seqlens) to the host and waits for the stream.
 *   - Sizes and strides are in ELEMENTS of the named dtype.  A "row" is one
 *     token (prefill) or one sequence (decode).  Within a row, head h of a
 *     [rows, H, D] operand starts at element h*D and is contiguous.
 *   - Input buffers are never written.  The state pool is updated in place.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     violation the call returns a negative code, enqueues nothing, and
 *     gdn_last_error() describes the problem (thread-local, prefixed with the
 *     entry point's name).  GDN_ERR_HIP means a launch failed.
 *   - Supported head sizes: Dk in {16, 32, 64, 128, 256}; any Dv >= 1.
 *     Pointers must be aligned to their element size and the state pool to
 *     16 bytes.  q/k are read with vector loads when every head start is
 *     aligned to 4 elements, with scalar loads otherwise.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GDN_F32 = 0, GDN_F16 = 1, GDN_BF16 = 2 } gdn_dtype;

enum {
  GDN_OK = 0,
  GDN_ERR_ARG = -1,    /* bad scalar argument, null pointer or misalignment */
  GDN_ERR_DTYPE = -2,  /* unsupported dtype or dtype combination */
  GDN_ERR_SHAPE = -3,  /* Hv not a multiple of Hk, unsupported Dk, stride < width */
  GDN_ERR_SLOT = -4,   /* GDN_CHECK_SLOTS found a duplicate or out-of-range slot */
  GDN_ERR_HIP = -5     /* a kernel launch failed */
};

enum {
  GDN_L2NORM_QK = 1u << 0,           /* L2-normalise q and k per head, eps = l2_eps */
  GDN_CHECK_SLOTS = 1u << 1,         /* check the slot table first (reads it; waits) */
  GDN_PREFILL_SEQUENTIAL = 1u << 2,  /* prefill: force the token-sequential kernel */
  GDN_STATE_F16 = 1u << 3,           /* state pool stored as IEEE binary16 */
  GDN_STATE_BF16 = 1u << 4,          /* state pool stored as bfloat16 */
  GDN_NORM_SIGMOID = 1u << 5,        /* gated norm: sigmoid gate instead of silu */
  /* 1u << 6 is not used */
  GDN_BETA_ROUNDED = 1u << 7,        /* gate_beta/post_conv/prefill_packed: round sigmoid(b) to b's dtype */
  GDN_CONV_SILU = 1u << 8            /* conv1d: silu activation (else identity) */
};
/*
 * Slot check (flag GDN_CHECK_SLOTS).  vllm.cpp test_ops_gdn.cpp, "gdn packed
 * decode rejects duplicate and out-of-range live slots".  Before enqueueing
 * anything the call copies state_idx (prefill: also cu_seqlens) to the host,
 * in order after the work already on `stream`, waits for it, and returns
 * GDN_ERR_SLOT when a live slot is >= num_slots or named twice (prefill: any
 * negative slot too) and GDN_ERR_SHAPE when cu_seqlens does not run
 * non-decreasing from 0 to total_tokens.  It returns GDN_ERR_ARG while the
 * stream is being captured.  Without the flag the slot table is trusted
 * (see each entry point for what a bad entry does).
 *
 * State storage dtype (flags GDN_STATE_F16 / GDN_STATE_BF16, at most one;
 * default f32).  vllm.cpp test_ops_gdn.cpp: "CUDA gdn decode corner fallback
 * supports indexed compressed state", the packed-decode port's note that the
 * op reads and writes persistent state in its declared FP16/BF16/F32 storage
 * dtype, and "gdn indexed state I/O: dtype conversion".  A 16-bit state is
 * widened to f32 when read, every step is computed in f32, and the new state
 * is rounded to nearest-even when written back; slots that are not written
 * keep their bytes.
 */

/*
 * gdn_gate -- g[r, h] = softplus(alpha[r, h] + dt_bias[h]) * ssm_a[h].
 * Winery-Strata elementwise_parity.cpp, gdn_gate block.
 *   g        [rows, hv] f32 output, row stride g_row_stride (>= hv).
 *   alpha    [rows, hv] in alpha_dt (f32, f16 or bf16), row stride
 *            alpha_row_stride (>= hv).
 *   dt_bias  [hv] f32.   ssm_a [hv] f32 (= -exp(A_log); negative).
 * Computed in f32 with the x > 20 branch, so it is finite for any finite x.
 * rows == 0 enqueues nothing and returns GDN_OK.
 */
int gdn_gate(float* g, int64_t g_row_stride, const void* alpha, gdn_dtype alpha_dt,
             int64_t alpha_row_stride, const float* dt_bias, const float* ssm_a,
             int64_t rows, int64_t hv, hipStream_t stream);

/*
 * gdn_conv1d_fwd -- depthwise causal conv1d over sequences packed back to back
 * (vllm.cpp test_ops_gdn.cpp, "causal_conv1d_fwd: bias + initial state,
 * hand-computed", the short-sequence write-back case, the padded-row case
 * and the CUDA varlen cases).  For channel c of token t in sequence s:
 *   out[t][c] = act(bias[c] + sum_{j<K} weight[c][j] * window[j])
 * where window[K-1] is x[t][c] and window[0..K-2] the K-1 inputs before it in
 * the same sequence, taken from the state row before the sequence's first
 * token (zeros when has_initial_state[s] == 0); act = silu with
 * GDN_CONV_SILU, else identity.  Afterwards the state row holds the last
 * K-1 raw inputs of (old window, the sequence's tokens): a sequence shorter
 * than K-1 shifts the old window left (zeros without an initial state).
 *   out          [total_tokens, channels] contiguous, out_dt (f32 or x_dt).
 *   x            row t at x + t * x_row_stride (>= channels), x_dt.
 *   weight       [channels, width] in x_dt;  bias [channels] in x_dt or NULL.
 *   conv_state   [num_slots, channels, state_len] (state_len >= width-1;
 *                only the leading width-1 entries are read or written, so a
 *                widened cache keeps its extra columns), f32 or GDN_STATE_F16
 *                / GDN_STATE_BF16; NULL allowed when width == 1.
 *   state_idx    [num_seqs] slot per sequence, or NULL (slot s).
 *   has_initial_state  [num_seqs] int8, or NULL (all 1).
 *   cu_seqlens   [num_seqs + 1] int32 as for gdn_prefill_varlen (read on the
 *                device; checked with GDN_CHECK_SLOTS, as are the slots).
 *   width        1..8 (width 1 keeps no state: conv_state, state_idx and
 *                num_slots are then unused).  flags: GDN_CONV_SILU,
 *                GDN_CHECK_SLOTS, GDN_STATE_*.
 * Unchecked (no GDN_CHECK_SLOTS), a sequence whose slot lies outside
 * [0, num_slots) gets NaN in every output row and keeps no state (width >= 2).
 * num_seqs == 0 enqueues nothing.
 */
int gdn_conv1d_fwd(void* out, gdn_dtype out_dt, const void* x, gdn_dtype x_dt,
                   int64_t x_row_stride, const void* weight, const void* bias,
                   void* conv_state, int64_t state_len, int64_t num_slots,
                   const int32_t* state_idx, const int8_t* has_initial_state,
                   const int32_t* cu_seqlens, int64_t num_seqs, int64_t total_tokens,
                   int64_t channels, int64_t width, uint32_t flags, hipStream_t stream);

/*
 * gdn_conv1d_update -- one token per row through the conv, rolling each
 * row's state (vllm.cpp test_ops_gdn.cpp, "causal_conv1d_update: bias +
 * rolling state", the indexed in-place and widened-cache cases):
 *   out[r][c] = act(bias[c] + sum_{j<K-1} weight[c][j] * state[j] +
 *                   weight[c][K-1] * x[r][c]),
 * then the state row shifts left by one and takes x[r][c] last.
 *   out        [batch, channels] contiguous, out_dt.
 *   x          row r at x + r * x_row_stride, x_dt.
 *   conv_state as for gdn_conv1d_fwd; state_idx [batch] or NULL (row r).
 *              A negative slot leaves that row's output and every state
 *              untouched; an out-of-range slot writes NaN and touches no
 *              state (GDN_CHECK_SLOTS rejects both duplicates and it).
 * batch == 0 enqueues nothing.
 */
int gdn_conv1d_update(void* out, gdn_dtype out_dt, const void* x, gdn_dtype x_dt,
                      int64_t x_row_stride, const void* weight, const void* bias,
                      void* conv_state, int64_t state_len, int64_t num_slots,
                      const int32_t* state_idx, int64_t batch, int64_t channels, int64_t width,
                      uint32_t flags, hipStream_t stream);

/*
 * gdn_gate_beta -- g and beta from the raw projections a and b (vllm.cpp
 * test_ops_gdn.cpp, GdnGBeta and the packed in_proj_ba case):
 *   g[r][h]    = softplus(a[r][h] + dt_bias[h]) * ssm_a[h]      (as gdn_gate)
 *   beta[r][h] = sigmoid(b[r][h]) in f32; with GDN_BETA_ROUNDED rounded
 *                through ab_dt (the packed decode's rule).
 *   g, beta    [rows, hv] f32 outputs, row stride out_row_stride (>= hv).
 *   a_raw, b_raw  [rows, hv] in ab_dt with their own row strides (>= hv):
 *                 e.g. column views of one merged [rows, 2*hv] b|a row.
 *   dt_bias, ssm_a  [hv] f32.
 * rows == 0 enqueues nothing.
 */
int gdn_gate_beta(float* g, float* beta, int64_t out_row_stride, const void* a_raw,
                  const void* b_raw, gdn_dtype ab_dt, int64_t a_row_stride,
                  int64_t b_row_stride, const float* dt_bias, const float* ssm_a, int64_t rows,
                  int64_t hv, uint32_t flags, hipStream_t stream);

/*
 * gdn_post_conv -- the front-end after the causal conv (vllm.cpp
 * test_ops_gdn.cpp, "gdn_post_conv fused == composed"): token t's conv row
 * (conv_dt, row stride conv_row_stride >= 2*hk*dk + hv*dv) holds q in columns
 * [0, hk*dk), k in [hk*dk, 2*hk*dk), v in [2*hk*dk, 2*hk*dk + hv*dv).
 *   q_out, k_out [T, hk, dk] contiguous, out_dt: q and k L2-normalised per
 *                head with l2_eps inside the root (no scale).
 *   v_out        [T, hv, dv] contiguous, out_dt: v converted.
 *   g_out, beta_out  [T, hv] f32 contiguous: as gdn_gate_beta from a_raw /
 *                b_raw (ab_dt, own row strides); flags: GDN_BETA_ROUNDED.
 * gdn_decode and gdn_prefill_varlen can read the conv rows directly (q, k, v
 * as row-strided views, norm in-kernel), so this pass is for callers that
 * want q, k, v materialised.  total_tokens == 0 enqueues nothing.
 */
int gdn_post_conv(void* q_out, void* k_out, void* v_out, gdn_dtype out_dt, float* g_out,
                  float* beta_out, const void* conv, gdn_dtype conv_dt, int64_t conv_row_stride,
                  const void* a_raw, const void* b_raw, gdn_dtype ab_dt, int64_t a_row_stride,
                  int64_t b_row_stride, const float* dt_bias, const float* ssm_a,
                  int64_t total_tokens, int64_t hk, int64_t hv, int64_t dk, int64_t dv,
                  float l2_eps, uint32_t flags, hipStream_t stream);

/*
 * gdn_decode -- one token for each of `batch` sequences, gate fused, states
 * updated in place in a slot-indexed pool.
 * vllm.cpp test_ops_gdn.cpp: "gdn decode: hand-computed single step" (the
 * step), "indexed in-place == compact reference" (slot addressing),
 * PackedDecodeReference (row-strided packed q|k|v, fused gate, q/k norm,
 * slot < 0 gives a zero output row).
 *   out        [batch, hv, dv] contiguous, out_dt (f32, or the input dtype).
 *   q, k       [batch, hk, dk] in in_dt with row strides q_row_stride,
 *              k_row_stride (>= hk*dk).  v: [batch, hv, dv], v_row_stride
 *              (>= hv*dv).  A packed q|k|v row is passed as three pointers
 *              into the same buffer with the same row stride.
 *   alpha      [batch, hv] in alpha_dt, row stride alpha_row_stride.
 *   dt_bias, ssm_a  [hv] f32.   beta [batch, hv] f32 (post-sigmoid),
 *              row stride beta_row_stride (gdn_decode_packed takes the raw
 *              projection b instead).
 *   state_pool [num_slots, hv, dv, dk] f32 (or binary16 / bfloat16 with
 *              GDN_STATE_F16 / GDN_STATE_BF16), read and written in place.
 *   state_idx  [batch] int32: row b uses slot state_idx[b].  A negative
 *              index marks a padded row: its output row is written as zeros
 *              and no state is touched.  An index >= num_slots is a caller
 *              error; such a row's output is written as NaN and no state is
 *              touched.  Two rows naming the same slot race (undefined).
 *   scale      > 0 and finite (usually 1/sqrt(dk)).
 *   flags      GDN_L2NORM_QK to normalise q and k with l2_eps; GDN_CHECK_SLOTS
 *              to validate state_idx first (negative entries allowed); at most
 *              one of GDN_STATE_F16, GDN_STATE_BF16.
 * batch == 0 enqueues nothing and returns GDN_OK.
 */
int gdn_decode(void* out, gdn_dtype out_dt, const void* q, const void* k, const void* v,
               gdn_dtype in_dt, int64_t q_row_stride, int64_t k_row_stride,
               int64_t v_row_stride, const void* alpha, gdn_dtype alpha_dt,
               int64_t alpha_row_stride, const float* dt_bias, const float* ssm_a,
               const float* beta, int64_t beta_row_stride, void* state_pool,
               int64_t num_slots, const int32_t* state_idx, int64_t batch, int64_t hk,
               int64_t hv, int64_t dk, int64_t dv, float scale, float l2_eps,
               uint32_t flags, hipStream_t stream);

/*
 * gdn_decode_packed -- gdn_decode from the raw gate projections a and b, as
 * the packed decode op takes them (vllm.cpp test_ops_gdn.cpp,
 * PackedDecodeReference and the packed in_proj_ba case): the step uses
 * g = softplus(a + dt_bias) * ssm_a and beta = sigmoid(b), the sigmoid
 * computed in f32 and rounded through ab_dt.
 *   a_raw, b_raw  [batch, hv] in ab_dt (f32, f16 or bf16) with their own row
 *              strides (>= hv): e.g. the a and b column views of one merged
 *              b|a projection row.
 *   every other argument as for gdn_decode (q, k, v may be views into the
 *   conv output row: q | k | v with its row stride).
 */
int gdn_decode_packed(void* out, gdn_dtype out_dt, const void* q, const void* k, const void* v,
                      gdn_dtype in_dt, int64_t q_row_stride, int64_t k_row_stride,
                      int64_t v_row_stride, const void* a_raw, const void* b_raw,
                      gdn_dtype ab_dt, int64_t a_row_stride, int64_t b_row_stride,
                      const float* dt_bias, const float* ssm_a, void* state_pool,
                      int64_t num_slots, const int32_t* state_idx, int64_t batch, int64_t hk,
                      int64_t hv, int64_t dk, int64_t dv, float scale, float l2_eps,
                      uint32_t flags, hipStream_t stream);

/*
 * gdn_decode_gated_norm -- gdn_decode followed, in the same kernel, by the
 * gated RMSNorm of each (row, v-head) output (see gdn_rmsnorm_gated):
 *   out[b][h][i] = o[i] / sqrt(mean_i o^2 + norm_eps) * norm_w[i] * act(z[b][h][i])
 * where o is the step's f32 output before any rounding.  vllm.cpp
 * test_ops_gdn.cpp, "rmsnorm_gated: norm-then-gate, silu and sigmoid
 * activations" and the rank-3 padded-row gate case (the gate is the z slice
 * of a wider projection row).
 *   all arguments of gdn_decode, plus
 *   norm_z     [batch, hv, dv] gate in in_dt; row b's head h starts at
 *              element b * norm_z_row_stride + h * dv (stride >= hv*dv, so a
 *              padded row of a wider buffer can be passed).  Never written.
 *   norm_w     [dv] weight in in_dt.
 *   norm_eps   >= 0 and finite, added to the mean square.
 *   flags      as gdn_decode, plus GDN_NORM_SIGMOID for a sigmoid gate
 *              (default silu(z) = z * sigmoid(z)).
 * Padded rows (negative slot) are written as zeros; rows with an
 * out-of-range slot as NaN.  Each (row, v-head) is one workgroup of at most
 * 8 waves, so dv <= 256 at dk = 128 (dk = 256: 128; dk = 16, 32, 64: 512);
 * larger dv returns GDN_ERR_SHAPE.
 */
int gdn_decode_gated_norm(void* out, gdn_dtype out_dt, const void* q, const void* k,
                          const void* v, gdn_dtype in_dt, int64_t q_row_stride,
                          int64_t k_row_stride, int64_t v_row_stride, const void* alpha,
                          gdn_dtype alpha_dt, int64_t alpha_row_stride, const float* dt_bias,
                          const float* ssm_a, const float* beta, int64_t beta_row_stride,
                          void* state_pool, int64_t num_slots, const int32_t* state_idx,
                          int64_t batch, int64_t hk, int64_t hv, int64_t dk, int64_t dv,
                          float scale, float l2_eps, const void* norm_z,
                          int64_t norm_z_row_stride, const void* norm_w, float norm_eps,
                          uint32_t flags, hipStream_t stream);

/*
 * gdn_rmsnorm_gated -- gated RMSNorm over [rows, hv, dv] (vllm.cpp
 * test_ops_gdn.cpp, "rmsnorm_gated: norm-then-gate, silu and sigmoid
 * activations", the CPU-vs-CUDA rmsnorm_gated cases and the rank-3
 * padded-row gate case):
 *   out[t][h][i] = x[t][h][i] / sqrt(mean_i x[t][h][i]^2 + eps) * norm_w[i]
 *                  * act(z[t][h][i]),   act = silu, or sigmoid with
 *                  GDN_NORM_SIGMOID.
 * The variance is a mean over dv; normalise first, then gate.
 *   out     [rows, hv, dv] contiguous, out_dt (f32 or x_dt).
 *   x       [rows, hv, dv] contiguous in x_dt (e.g. the prefill output).
 *   z       gate in x_dt: token t's head h starts at t * z_row_stride + h*dv
 *           (z_row_stride >= hv*dv); the buffer must hold
 *           (rows - 1) * z_row_stride + hv*dv elements.  Never written.
 *   norm_w  [dv] in x_dt.
 *   eps     >= 0 and finite.
 * Computed in f32, output rounded to nearest-even.  rows == 0 enqueues
 * nothing.  Fast path: with N = 16 bytes of x_dt elements (8 for f16/bf16, 4
 * for f32), dv / N a power of two <= 64, z_row_stride a multiple of N and
 * every pointer 16-byte aligned; any other layout takes a slower
 * wave-per-row kernel.
 */
int gdn_rmsnorm_gated(void* out, gdn_dtype out_dt, const void* x, gdn_dtype x_dt,
                      const void* z, int64_t z_row_stride, const void* norm_w, int64_t rows,
                      int64_t hv, int64_t dv, float eps, uint32_t flags, hipStream_t stream);

/*
 * gdn_prefill_varlen_workspace_size -- bytes of device workspace that
 * gdn_prefill_varlen (and gdn_prefill_varlen_aux) needs for these sizes and
 * flags (0 if none).  The chunked path (bf16/fp16 inputs, dk = 128, dv a
 * multiple of 16) keeps one 25,600-byte record per (64-token chunk, v-head):
 * about (total_tokens / 64 + num_seqs) * hv * 25,600 bytes, plus about 12
 * bytes per sequence, plus for the (at most two) longest sequences it may
 * split into segments up to 8 f32 states of dv x dk per v-head (fewer when
 * total_tokens is small); the token-sequential path needs none.  Whether a call takes the
 * chunked path also depends on its pointers (16-byte aligned q/k/v rows,
 * strides multiples of 8 elements): with a smaller workspace it fails rather
 * than falling back.
 */
size_t gdn_prefill_varlen_workspace_size(int64_t total_tokens, int64_t num_seqs, int64_t hk,
                                         int64_t hv, int64_t dk, int64_t dv, gdn_dtype in_dt,
                                         uint32_t flags);

/*
 * gdn_prefill_varlen -- the recurrence over many sequences packed back to back.
 * vllm.cpp test_ops_gdn.cpp: the 3-token prefill table, "multi-sequence
 * varlen equals independent runs" (cu_seqlens = query_start_loc), "T=1
 * equals decode", and the state gather/scatter cases (initial state read from
 * a cache slot, fresh sequences start from zeros, final state written back).
 *   out          [total_tokens, hv, dv] contiguous, out_dt.
 *   q, k, v      as for gdn_decode with one row per token.
 *   g            [total_tokens, hv] f32 (from gdn_gate), row stride g_row_stride.
 *   beta         [total_tokens, hv] f32, row stride beta_row_stride.
 *   state_pool   [num_slots, hv, dv, dk] f32 (binary16 / bfloat16 with
 *                GDN_STATE_F16 / GDN_STATE_BF16).  Sequence s starts from
 *                pool[slot] (slot = state_idx[s], or s when state_idx is
 *                NULL) when has_initial_state[s] != 0 (NULL: all nonzero),
 *                else from zeros without reading the slot, and its final
 *                state is written to pool[slot].  Slots must be distinct and
 *                in [0, num_slots): checked with GDN_CHECK_SLOTS; otherwise
 *                a sequence whose slot is out of range gets NaN outputs and
 *                no state access, and two sequences naming one slot race.
 *   cu_seqlens   [num_seqs + 1] int32, cu_seqlens[0] = 0, non-decreasing,
 *                cu_seqlens[num_seqs] = total_tokens.  Read on the device,
 *                where every range is clamped to [0, total_tokens); checked
 *                with GDN_CHECK_SLOTS.
 *                A zero-length sequence passes its state through unchanged.
 *   workspace    device buffer of at least
 *                gdn_prefill_varlen_workspace_size(...) bytes (may be NULL
 *                when that size is 0).
 *   flags        GDN_L2NORM_QK; GDN_CHECK_SLOTS; GDN_PREFILL_SEQUENTIAL
 *                forces the token-sequential kernel instead of the chunked
 *                one; at most one of GDN_STATE_F16, GDN_STATE_BF16.
 * num_seqs == 0 enqueues nothing and returns GDN_OK.
 * Streams: every kernel runs on `stream` (gdn_prefill_varlen_aux may also
 * use a second stream the caller passes).  The library owns no stream and
 * holds no lock across launches; calls on different streams run
 * concurrently, each in its own workspace.
 */
int gdn_prefill_varlen(void* out, gdn_dtype out_dt, const void* q, const void* k,
                       const void* v, gdn_dtype in_dt, int64_t q_row_stride,
                       int64_t k_row_stride, int64_t v_row_stride, const float* g,
                       int64_t g_row_stride, const float* beta, int64_t beta_row_stride,
                       void* state_pool, int64_t num_slots, const int32_t* state_idx,
                       const int8_t* has_initial_state, const int32_t* cu_seqlens,
                       int64_t num_seqs, int64_t total_tokens, int64_t hk, int64_t hv,
                       int64_t dk, int64_t dv, float scale, float l2_eps, uint32_t flags,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gdn_prefill_varlen_aux -- gdn_prefill_varlen with a second stream of the
 * caller's, aux_stream, for the split schedule: when the lengths are skewed,
 * the records and walks of the shorter sequences run on aux_stream beside the
 * longest sequences' walks on `stream`, forked from and joined back into
 * `stream` with two events (created per host thread and device on first use
 * and kept for the life of the process), so later work on `stream` sees
 * every result and `aux_stream` is left with no pending dependency on this
 * call's later work.  aux_stream must be on the same device as `stream`;
 * NULL, equal to `stream`, on another device, or while `stream` is being
 * captured, the call runs on `stream` alone exactly as gdn_prefill_varlen.
 * Two calls that share aux_stream are serialised on it.
 */
int gdn_prefill_varlen_aux(void* out, gdn_dtype out_dt, const void* q, const void* k,
                           const void* v, gdn_dtype in_dt, int64_t q_row_stride,
                           int64_t k_row_stride, int64_t v_row_stride, const float* g,
                           int64_t g_row_stride, const float* beta, int64_t beta_row_stride,
                           void* state_pool, int64_t num_slots, const int32_t* state_idx,
                           const int8_t* has_initial_state, const int32_t* cu_seqlens,
                           int64_t num_seqs, int64_t total_tokens, int64_t hk, int64_t hv,
                           int64_t dk, int64_t dv, float scale, float l2_eps, uint32_t flags,
                           void* workspace, size_t workspace_bytes, hipStream_t stream,
                           hipStream_t aux_stream);

/*
 * gdn_prefill_varlen_gated -- gdn_prefill_varlen_aux with the gate fused, as
 * gdn_decode fuses it: no g array; the kernels form
 * g = softplus(alpha + dt_bias) * ssm_a for each (token, v-head) with the
 * arithmetic of gdn_gate, so the result is bit-identical to gdn_gate followed
 * by gdn_prefill_varlen_aux (Winery-Strata elementwise_parity.cpp, the
 * gdn_gate block; vllm.cpp test_ops_gdn.cpp, GdnPrefill's inputs).
 *   alpha      [total_tokens, hv] in alpha_dt (f32, f16 or bf16), row stride
 *              alpha_row_stride (>= hv).   dt_bias, ssm_a  [hv] f32.
 *   beta       [total_tokens, hv] f32 post-sigmoid, row stride beta_row_stride.
 *   every other argument as for gdn_prefill_varlen_aux (aux_stream may be
 *   NULL), the same workspace size.
 */
int gdn_prefill_varlen_gated(void* out, gdn_dtype out_dt, const void* q, const void* k,
                             const void* v, gdn_dtype in_dt, int64_t q_row_stride,
                             int64_t k_row_stride, int64_t v_row_stride, const void* alpha,
                             gdn_dtype alpha_dt, int64_t alpha_row_stride, const float* dt_bias,
                             const float* ssm_a, const float* beta, int64_t beta_row_stride,
                             void* state_pool, int64_t num_slots, const int32_t* state_idx,
                             const int8_t* has_initial_state, const int32_t* cu_seqlens,
                             int64_t num_seqs, int64_t total_tokens, int64_t hk, int64_t hv,
                             int64_t dk, int64_t dv, float scale, float l2_eps, uint32_t flags,
                             void* workspace, size_t workspace_bytes, hipStream_t stream,
                             hipStream_t aux_stream);

/*
 * gdn_prefill_varlen_gated_norm -- gdn_prefill_varlen_gated followed, on the
 * same stream, by the gated RMSNorm of gdn_rmsnorm_gated over the output in
 * place (vllm.cpp test_ops_gdn.cpp, "rmsnorm_gated: norm-then-gate, silu and
 * sigmoid activations" and "rank-3 padded-row strided gate matches
 * contiguous"):
 *   out[t][h][i] = o / sqrt(mean_i(o^2) + norm_eps) * norm_w[i] * act(z),
 * act = silu, or sigmoid with GDN_NORM_SIGMOID, from the output as stored.
 * The result is bit-identical to gdn_prefill_varlen_gated then
 * gdn_rmsnorm_gated(out, out, ...).  The norm is a second pass over out, not
 * part of the walk's store: a v-head's Dv output rows are split between two
 * workgroups of the walk, and a row's mean of squares would need an exchange
 * between them at every chunk.
 *   norm_z     [total_tokens, hv, dv] in in_dt, row stride norm_z_row_stride
 *              (>= hv*dv; a padded view of a wider row is fine).
 *   norm_w     [dv] in in_dt.   norm_eps  finite, >= 0.
 *   out_dt     must equal in_dt (norm_z and norm_w share it).
 *   flags      as gdn_prefill_varlen, plus GDN_NORM_SIGMOID.
 *   every other argument as for gdn_prefill_varlen_gated (aux_stream may be
 *   NULL), the same workspace size.  The norm's arguments are checked before
 *   anything is enqueued; a failure of either launch returns GDN_ERR_HIP.
 */
int gdn_prefill_varlen_gated_norm(void* out, gdn_dtype out_dt, const void* q, const void* k,
                                  const void* v, gdn_dtype in_dt, int64_t q_row_stride,
                                  int64_t k_row_stride, int64_t v_row_stride, const void* alpha,
                                  gdn_dtype alpha_dt, int64_t alpha_row_stride,
                                  const float* dt_bias, const float* ssm_a, const float* beta,
                                  int64_t beta_row_stride, void* state_pool, int64_t num_slots,
                                  const int32_t* state_idx, const int8_t* has_initial_state,
                                  const int32_t* cu_seqlens, int64_t num_seqs,
                                  int64_t total_tokens, int64_t hk, int64_t hv, int64_t dk,
                                  int64_t dv, float scale, float l2_eps, const void* norm_z,
                                  int64_t norm_z_row_stride, const void* norm_w, float norm_eps,
                                  uint32_t flags, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, hipStream_t aux_stream);

/*
 * gdn_prefill_varlen_packed -- the prefill fed by the front-end's raw
 * projections (vllm.cpp test_ops_gdn.cpp, "gdn_post_conv fused == composed"
 * and the packed in_proj_ba case): q, k, v may be views into the conv output
 * rows (q | k | v with its row stride; normalised in the kernels with
 * GDN_L2NORM_QK), and g and beta are formed per (token, v-head) from the raw
 * a and b: g = softplus(a + dt_bias) * ssm_a, beta = sigmoid(b) in f32, with
 * GDN_BETA_ROUNDED rounded through ab_dt -- bit-identical to gdn_gate_beta
 * (same flag) followed by gdn_prefill_varlen_aux.  Nothing but the outputs
 * and final states is written: no q, k, v, g or beta array is formed.
 *   a_raw, b_raw  [total_tokens, hv] in ab_dt with their own row strides
 *              (>= hv): e.g. the a and b column views of one merged b|a row.
 *   dt_bias, ssm_a  [hv] f32.
 *   flags      as gdn_prefill_varlen, plus GDN_BETA_ROUNDED.
 *   every other argument as for gdn_prefill_varlen_aux.
 */
int gdn_prefill_varlen_packed(void* out, gdn_dtype out_dt, const void* q, const void* k,
                              const void* v, gdn_dtype in_dt, int64_t q_row_stride,
                              int64_t k_row_stride, int64_t v_row_stride, const void* a_raw,
                              const void* b_raw, gdn_dtype ab_dt, int64_t a_row_stride,
                              int64_t b_row_stride, const float* dt_bias, const float* ssm_a,
                              void* state_pool, int64_t num_slots, const int32_t* state_idx,
                              const int8_t* has_initial_state, const int32_t* cu_seqlens,
                              int64_t num_seqs, int64_t total_tokens, int64_t hk, int64_t hv,
                              int64_t dk, int64_t dv, float scale, float l2_eps, uint32_t flags,
                              void* workspace, size_t workspace_bytes, hipStream_t stream,
                              hipStream_t aux_stream);

/*
 * gdn_prefill_varlen_noalloc -- gdn_prefill_varlen with no workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It takes
 * every other argument of gdn_prefill_varlen with the same meaning, layout
 * and errors, runs the same kernels, and allocates nothing: the chunked path's
 * per-call records live in a fixed scratch array of
 * GDN_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends (its address is looked up on the first call on a
 * device, with that device current).
 *   Limit: sizes whose gdn_prefill_varlen_workspace_size exceeds
 *   GDN_NOALLOC_SCRATCH_BYTES return GDN_ERR_SHAPE and enqueue nothing (128
 *   MiB holds e.g. one 8192-token sequence at hv = 32, dv = 128).
 *   Sharing: every call on a device uses that device's one array, and the
 *   whole call stays on `stream`; calls that overlap on one device -- on
 *   different streams or host threads, or graph replays running
 *   concurrently -- race on it and give undefined results.  Calls ordered on
 *   one stream are safe; each call rewrites what it reads.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

int gdn_prefill_varlen_noalloc(void* out, gdn_dtype out_dt, const void* q, const void* k,
                               const void* v, gdn_dtype in_dt, int64_t q_row_stride,
                               int64_t k_row_stride, int64_t v_row_stride, const float* g,
                               int64_t g_row_stride, const float* beta,
                               int64_t beta_row_stride, void* state_pool, int64_t num_slots,
                               const int32_t* state_idx, const int8_t* has_initial_state,
                               const int32_t* cu_seqlens, int64_t num_seqs,
                               int64_t total_tokens, int64_t hk, int64_t hv, int64_t dk,
                               int64_t dv, float scale, float l2_eps, uint32_t flags,
                               hipStream_t stream);

/* Message for the last error returned on this thread ("" if none). */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
