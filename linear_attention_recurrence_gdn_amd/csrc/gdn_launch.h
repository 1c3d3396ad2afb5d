// gdn_launch.h -- internal interface between the C ABI (gdn_api.hip) and the
// kernel launchers.  Arguments are validated before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct GateArgs {
  float* g;
  int64_t g_rs;
  const void* alpha;
  int alpha_dt;
  int64_t alpha_rs;
  const float* dt_bias;
  const float* ssm_a;
  int64_t rows;
  int64_t hv;
  // optional beta from the raw projection b (same dtype as alpha)
  const void* b;       // nullptr: no beta
  int64_t b_rs;
  float* beta;
  int64_t beta_rs;
  int round_beta;      // sigmoid rounded through b's dtype
};

// Post-conv front-end: conv output rows [T, 2*hk*dk + hv*dv (+ padding)] ->
// q, k normalised [T, hk, dk], v [T, hv, dv] (contiguous, out_dt).
struct PostConvArgs {
  void* q;
  void* k;
  void* v;
  int out_dt;
  const void* conv;
  int conv_dt;
  int64_t conv_rs;
  int64_t T;
  int hk, hv, dk, dv;
  float l2_eps;
};

struct DecodeArgs {
  void* out;
  int out_dt;
  const void* q;
  const void* k;
  const void* v;
  int in_dt;
  int64_t q_rs, k_rs, v_rs;
  int qk_vec;  // q/k head starts are 4-element aligned: vector loads
  const void* alpha;
  int alpha_dt;
  int64_t alpha_rs;
  const float* dt_bias;
  const float* ssm_a;
  const void* beta;  // f32 post-sigmoid, or (beta_raw) the raw b in alpha_dt
  int64_t beta_rs;
  int beta_raw;      // beta = sigmoid(b) rounded through alpha_dt
  void* pool;     // [slots, hv, dv, dk] in state_dt
  int state_dt;   // kF32, kF16 or kBF16 storage; the step is computed in f32
  int64_t num_slots;
  const int32_t* idx;
  int64_t batch;
  int hk, hv, dk, dv;
  float scale, l2_eps;
  int l2norm;
  // gated RMSNorm epilogue (norm_z == nullptr: none): out = o / rms(o) * w * act(z)
  const void* norm_z;    // [batch, hv, dv] in in_dt, token row stride norm_z_rs
  int64_t norm_z_rs;
  const void* norm_w;    // [dv] in in_dt
  float norm_eps;
  int norm_sigmoid;      // act: 0 silu, 1 sigmoid
};

// Gated RMSNorm over [rows, hv, dv]: x, z and w share x_dt.
struct NormArgs {
  void* out;
  int out_dt;
  const void* x;       // [rows, hv, dv] contiguous
  int x_dt;
  const void* z;       // token t's head h at z[t * z_rs + h * dv]
  int64_t z_rs;
  const void* w;       // [dv]
  int64_t rows;
  int hv, dv;
  float eps;
  int sigmoid;
};

// Depthwise causal conv1d (forward over packed sequences, or single-token update).
struct ConvArgs {
  void* out;             // [T or batch, C] contiguous, out_dt
  int out_dt;
  const void* x;         // row t at x + t * x_rs, x_dt
  int x_dt;
  int64_t x_rs;
  const void* w;         // [C, K] in x_dt
  const void* bias;      // [C] in x_dt, or nullptr
  void* state;           // [num_slots, C, state_len] in state_dt (leading K-1 used)
  int state_dt;
  int64_t state_len;
  int64_t num_slots;
  const int32_t* idx;      // [n] slot per sequence / row, or nullptr (s)
  const int8_t* has_init;  // forward: [n] or nullptr (all 1)
  const int32_t* cu;       // forward: [n + 1]
  int64_t n;               // sequences (forward) or rows (update)
  int64_t T;               // tokens (forward)
  int64_t C;
  int K;
  int silu;
};

struct PrefillArgs {
  void* out;
  int out_dt;
  const void* q;
  const void* k;
  const void* v;
  int in_dt;
  int64_t q_rs, k_rs, v_rs;
  int qk_vec;
  const float* g;       // [T, hv] f32, or null: formed from alpha below
  int64_t g_rs;
  const void* beta;     // [T, hv] f32 post-sigmoid, or (beta_raw) the raw b in alpha_dt
  int64_t beta_rs;
  // the gate fused (alpha != null): g = softplus(alpha + dt_bias) * ssm_a per
  // (token, v-head), exactly as gate_kernel forms it
  const void* alpha;
  int alpha_dt;
  int64_t alpha_rs;
  const float* dt_bias;
  const float* ssm_a;
  int beta_raw;         // beta = sigmoid(b) of the raw b (in alpha_dt) ...
  int round_beta;       // ... rounded through alpha_dt
  void* pool;     // [slots, hv, dv, dk] in state_dt
  int state_dt;
  int64_t num_slots;
  const int32_t* idx;       // may be null: slot s
  const int8_t* has_init;   // may be null: all 1
  const int32_t* cu;
  int64_t num_seqs;
  int64_t total_tokens;
  int hk, hv, dk, dv;
  float scale, l2_eps;
  int l2norm;
};

hipError_t launch_gate(const GateArgs& a, hipStream_t stream);
hipError_t launch_post_conv(const PostConvArgs& a, hipStream_t stream);
constexpr int kConvMaxK = 8;
hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t stream);
hipError_t launch_conv_update(const ConvArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// the fused-norm decode runs one workgroup (at most 16 waves) per (row,
// v-head): the largest dv it takes at this dk
int decode_norm_max_dv(int dk);
hipError_t launch_rmsnorm_gated(const NormArgs& a, hipStream_t stream);
hipError_t launch_prefill_sequential(const PrefillArgs& a, hipStream_t stream);

// Chunked prefill (MFMA).  Returns hipErrorNotSupported when the shape or
// dtype has no chunked kernel (the caller then uses the sequential one).
bool chunked_supported(int in_dt, int out_dt, int64_t hv, int dk, int dv);
// the chunked kernels stage q/k/v rows with 16-byte loads
bool chunked_layout_ok(const void* q, const void* k, const void* v, int64_t q_rs, int64_t k_rs,
                       int64_t v_rs);
size_t chunked_workspace_bytes(int64_t total_tokens, int64_t num_seqs, int hv, int dk, int dv);
// `aux` (may be null): the caller's second stream for the split schedule.
hipError_t launch_prefill_chunked(const PrefillArgs& a, void* ws, size_t ws_bytes,
                                  hipStream_t stream, hipStream_t aux);

}  // namespace gdn
