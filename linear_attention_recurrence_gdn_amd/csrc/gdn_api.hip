// gdn_api.hip -- the C ABI declared in include/gdn.h: host-side argument
// validation and dispatch to the kernel launchers.  Nothing here allocates
// device memory; only GDN_CHECK_SLOTS reads device data (the slot table and
// cu_seqlens, copied to the host in stream order) and so waits on the stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return GDN_OK;
}

bool valid_dt(int dt) { return dt == GDN_F32 || dt == GDN_F16 || dt == GDN_BF16; }
int elem_bytes(int dt) { return dt == GDN_F32 ? 4 : 2; }
bool supported_dk(int64_t dk) {
  return dk == 16 || dk == 32 || dk == 64 || dk == 128 || dk == 256;
}
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// q/k are read 4 elements at a time from every head start: vector loads when
// every head start is aligned to 4 elements, scalar loads otherwise.
bool qk_vector_ok(const void* q, const void* k, int in_dt, int64_t q_rs, int64_t k_rs) {
  const size_t vec = 4 * (size_t)elem_bytes(in_dt);
  return aligned(q, vec) && aligned(k, vec) && q_rs % 4 == 0 && k_rs % 4 == 0;
}

int check_qk(const char* op, const void* q, const void* k, int in_dt, int64_t q_rs,
             int64_t k_rs, int64_t hk, int64_t dk) {
  const size_t eb = (size_t)elem_bytes(in_dt);
  if (!aligned(q, eb) || !aligned(k, eb))
    return fail(GDN_ERR_ARG, "%s: q/k pointers must be aligned to their element size", op);
  if (q_rs < hk * dk || k_rs < hk * dk)
    return fail(GDN_ERR_SHAPE, "%s: q/k row stride (%lld, %lld) below hk*dk = %lld", op,
                (long long)q_rs, (long long)k_rs, (long long)(hk * dk));
  return GDN_OK;
}

int check_heads(const char* op, int64_t hk, int64_t hv, int64_t dk, int64_t dv) {
  if (hk <= 0 || hv <= 0 || dk <= 0 || dv <= 0)
    return fail(GDN_ERR_SHAPE, "%s: head counts and sizes must be positive", op);
  if (hv % hk != 0)
    return fail(GDN_ERR_SHAPE, "%s: Hv (%lld) must be a multiple of Hk (%lld)", op,
                (long long)hv, (long long)hk);
  if (!supported_dk(dk))
    return fail(GDN_ERR_SHAPE, "%s: Dk = %lld not supported (16, 32, 64, 128, 256)", op,
                (long long)dk);
  if (hv > (1 << 20) || dv > (1 << 20))
    return fail(GDN_ERR_SHAPE, "%s: Hv/Dv too large", op);
  return GDN_OK;
}

int check_scale(const char* op, float scale, float eps) {
  if (!(scale > 0.0f) || !isfinite(scale))
    return fail(GDN_ERR_ARG, "%s: scale must be set (finite and > 0), got %g", op,
                (double)scale);
  if (!(eps >= 0.0f) || !isfinite(eps))
    return fail(GDN_ERR_ARG, "%s: l2_eps must be finite and >= 0", op);
  return GDN_OK;
}

// storage dtype of the state pool from the flags, or -1 when both are set
int state_dtype(uint32_t flags) {
  const bool f16 = (flags & GDN_STATE_F16) != 0, bf16 = (flags & GDN_STATE_BF16) != 0;
  if (f16 && bf16) return -1;
  return f16 ? GDN_F16 : bf16 ? GDN_BF16 : GDN_F32;
}

// GDN_CHECK_SLOTS (vllm.cpp test_ops_gdn.cpp, the packed-decode case that
// rejects duplicate and out-of-range live slots): copy `n` int32 entries of
// device metadata to the host after the work already on `stream`, and wait.
int fetch_i32(const char* op, const int32_t* dev, int64_t n, std::vector<int32_t>& host,
              hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess)
    return fail(GDN_ERR_HIP, "%s: stream query failed: %s", op, hipGetErrorString(e));
  if (cs != hipStreamCaptureStatusNone)
    return fail(GDN_ERR_ARG, "%s: GDN_CHECK_SLOTS waits on the stream and cannot be captured",
                op);
  host.resize((size_t)n);
  e = hipMemcpyAsync(host.data(), dev, (size_t)n * sizeof(int32_t),
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess)
    return fail(GDN_ERR_HIP, "%s: reading device metadata failed: %s", op, hipGetErrorString(e));
  return GDN_OK;
}

// Live slots (>= 0; negative ones allowed only where they mark padded rows)
// must lie in [0, num_slots) and be distinct.
int check_slot_table(const char* op, const std::vector<int32_t>& idx, int64_t num_slots,
                     bool allow_negative) {
  std::vector<int32_t> live;
  live.reserve(idx.size());
  for (size_t i = 0; i < idx.size(); ++i) {
    const int32_t s = idx[i];
    if (s < 0 && allow_negative) continue;
    if (s < 0 || s >= num_slots)
      return fail(GDN_ERR_SLOT, "%s: row %zu names slot %d, outside [0, %lld)", op, i, (int)s,
                  (long long)num_slots);
    live.push_back(s);
  }
  std::sort(live.begin(), live.end());
  const auto d = std::adjacent_find(live.begin(), live.end());
  if (d != live.end())
    return fail(GDN_ERR_SLOT, "%s: slot %d is named by more than one row", op, (int)*d);
  return GDN_OK;
}

int hip_status(const char* op, hipError_t e) {
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: launch failed: %s", op, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* gdn_last_error(void) { return g_err; }

int gdn_gate(float* g, int64_t g_row_stride, const void* alpha, gdn_dtype alpha_dt,
             int64_t alpha_row_stride, const float* dt_bias, const float* ssm_a, int64_t rows,
             int64_t hv, hipStream_t stream) {
  const char* op = "gdn_gate";
  if (rows < 0 || hv <= 0) return fail(GDN_ERR_SHAPE, "%s: rows >= 0 and hv > 0 required", op);
  if (!valid_dt(alpha_dt)) return fail(GDN_ERR_DTYPE, "%s: unknown alpha dtype %d", op, alpha_dt);
  if (g_row_stride < hv || alpha_row_stride < hv)
    return fail(GDN_ERR_SHAPE, "%s: row strides must be >= hv", op);
  if (rows == 0) return ok();
  if (!g || !alpha || !dt_bias || !ssm_a) return fail(GDN_ERR_ARG, "%s: null pointer", op);
  gdn::GateArgs a{};
  a.g = g; a.g_rs = g_row_stride; a.alpha = alpha; a.alpha_dt = alpha_dt;
  a.alpha_rs = alpha_row_stride; a.dt_bias = dt_bias; a.ssm_a = ssm_a; a.rows = rows; a.hv = hv;
  return hip_status(op, gdn::launch_gate(a, stream));
}

int gdn_gate_beta(float* g, float* beta, int64_t out_row_stride, const void* a_raw,
                  const void* b_raw, gdn_dtype ab_dt, int64_t a_row_stride,
                  int64_t b_row_stride, const float* dt_bias, const float* ssm_a, int64_t rows,
                  int64_t hv, uint32_t flags, hipStream_t stream) {
  const char* op = "gdn_gate_beta";
  if (rows < 0 || hv <= 0) return fail(GDN_ERR_SHAPE, "%s: rows >= 0 and hv > 0 required", op);
  if (!valid_dt(ab_dt)) return fail(GDN_ERR_DTYPE, "%s: unknown a/b dtype %d", op, ab_dt);
  if (flags & ~(uint32_t)GDN_BETA_ROUNDED)
    return fail(GDN_ERR_ARG, "%s: unknown flags 0x%x", op, flags);
  if (out_row_stride < hv || a_row_stride < hv || b_row_stride < hv)
    return fail(GDN_ERR_SHAPE, "%s: row strides must be >= hv", op);
  if (rows == 0) return ok();
  if (!g || !beta || !a_raw || !b_raw || !dt_bias || !ssm_a)
    return fail(GDN_ERR_ARG, "%s: null pointer", op);
  const size_t eb = (size_t)elem_bytes(ab_dt);
  if (!aligned(a_raw, eb) || !aligned(b_raw, eb) || !aligned(g, 4) || !aligned(beta, 4))
    return fail(GDN_ERR_ARG, "%s: pointers must be aligned to their element size", op);
  gdn::GateArgs a{};
  a.g = g; a.g_rs = out_row_stride; a.alpha = a_raw; a.alpha_dt = ab_dt;
  a.alpha_rs = a_row_stride; a.dt_bias = dt_bias; a.ssm_a = ssm_a; a.rows = rows; a.hv = hv;
  a.b = b_raw; a.b_rs = b_row_stride; a.beta = beta; a.beta_rs = out_row_stride;
  a.round_beta = (flags & GDN_BETA_ROUNDED) ? 1 : 0;
  return hip_status(op, gdn::launch_gate(a, stream));
}

int gdn_post_conv(void* q_out, void* k_out, void* v_out, gdn_dtype out_dt, float* g_out,
                  float* beta_out, const void* conv, gdn_dtype conv_dt, int64_t conv_row_stride,
                  const void* a_raw, const void* b_raw, gdn_dtype ab_dt, int64_t a_row_stride,
                  int64_t b_row_stride, const float* dt_bias, const float* ssm_a,
                  int64_t total_tokens, int64_t hk, int64_t hv, int64_t dk, int64_t dv,
                  float l2_eps, uint32_t flags, hipStream_t stream) {
  const char* op = "gdn_post_conv";
  const int64_t T = total_tokens;
  if (T < 0) return fail(GDN_ERR_SHAPE, "%s: negative total_tokens", op);
  if (hk <= 0 || hv <= 0 || dk <= 0 || dv <= 0 || hv % hk != 0)
    return fail(GDN_ERR_SHAPE, "%s: positive sizes and Hv a multiple of Hk required", op);
  if (hk > (1 << 16) || hv > (1 << 20) || dk > (1 << 16) || dv > (1 << 20))
    return fail(GDN_ERR_SHAPE, "%s: head counts or sizes too large", op);
  if (!valid_dt(out_dt) || !valid_dt(conv_dt) || !valid_dt(ab_dt))
    return fail(GDN_ERR_DTYPE, "%s: unknown dtype", op);
  if (flags & ~(uint32_t)GDN_BETA_ROUNDED)
    return fail(GDN_ERR_ARG, "%s: unknown flags 0x%x", op, flags);
  if (!(l2_eps >= 0.0f) || !isfinite(l2_eps))
    return fail(GDN_ERR_ARG, "%s: l2_eps must be finite and >= 0", op);
  if (conv_row_stride < 2 * hk * dk + hv * dv)
    return fail(GDN_ERR_SHAPE, "%s: conv row stride below 2*Hk*Dk + Hv*Dv", op);
  if (a_row_stride < hv || b_row_stride < hv)
    return fail(GDN_ERR_SHAPE, "%s: a/b row strides must be >= hv", op);
  if (T == 0) return ok();
  if (!q_out || !k_out || !v_out || !g_out || !beta_out || !conv || !a_raw || !b_raw ||
      !dt_bias || !ssm_a)
    return fail(GDN_ERR_ARG, "%s: null pointer", op);
  const size_t eo = (size_t)elem_bytes(out_dt), ec = (size_t)elem_bytes(conv_dt),
               eab = (size_t)elem_bytes(ab_dt);
  if (!aligned(q_out, eo) || !aligned(k_out, eo) || !aligned(v_out, eo) || !aligned(conv, ec) ||
      !aligned(a_raw, eab) || !aligned(b_raw, eab) || !aligned(g_out, 4) || !aligned(beta_out, 4))
    return fail(GDN_ERR_ARG, "%s: pointers must be aligned to their element size", op);
  if (T >= ((int64_t)1 << 31)) return fail(GDN_ERR_SHAPE, "%s: total_tokens too large", op);
  gdn::PostConvArgs p{};
  p.q = q_out; p.k = k_out; p.v = v_out; p.out_dt = out_dt; p.conv = conv; p.conv_dt = conv_dt;
  p.conv_rs = conv_row_stride; p.T = T; p.hk = (int)hk; p.hv = (int)hv; p.dk = (int)dk;
  p.dv = (int)dv; p.l2_eps = l2_eps;
  const int rc = hip_status(op, gdn::launch_post_conv(p, stream));
  if (rc) return rc;
  gdn::GateArgs a{};
  a.g = g_out; a.g_rs = hv; a.alpha = a_raw; a.alpha_dt = ab_dt; a.alpha_rs = a_row_stride;
  a.dt_bias = dt_bias; a.ssm_a = ssm_a; a.rows = T; a.hv = hv;
  a.b = b_raw; a.b_rs = b_row_stride; a.beta = beta_out; a.beta_rs = hv;
  a.round_beta = (flags & GDN_BETA_ROUNDED) ? 1 : 0;
  return hip_status(op, gdn::launch_gate(a, stream));
}

}  // extern "C"

namespace {

int conv_common(const char* op, gdn_dtype out_dt, gdn_dtype x_dt, int64_t x_row_stride,
                int64_t state_len, int64_t num_slots, int64_t channels, int64_t width,
                uint32_t flags, uint32_t extra_flags) {
  if (!valid_dt(x_dt) || !valid_dt(out_dt)) return fail(GDN_ERR_DTYPE, "%s: unknown dtype", op);
  if (out_dt != GDN_F32 && out_dt != x_dt)
    return fail(GDN_ERR_DTYPE, "%s: out dtype must be f32 or the input dtype", op);
  if (flags & ~(uint32_t)(GDN_CONV_SILU | GDN_CHECK_SLOTS | GDN_STATE_F16 | GDN_STATE_BF16 |
                          extra_flags))
    return fail(GDN_ERR_ARG, "%s: unknown flags 0x%x", op, flags);
  if (state_dtype(flags) < 0)
    return fail(GDN_ERR_DTYPE, "%s: GDN_STATE_F16 and GDN_STATE_BF16 both set", op);
  if (channels <= 0 || channels > ((int64_t)65535 * 256))
    return fail(GDN_ERR_SHAPE, "%s: channels must be in [1, %d]", op, 65535 * 256);
  if (width < 1 || width > gdn::kConvMaxK)
    return fail(GDN_ERR_SHAPE, "%s: width %lld not in [1, %d]", op, (long long)width,
                gdn::kConvMaxK);
  if (x_row_stride < channels) return fail(GDN_ERR_SHAPE, "%s: x row stride below channels", op);
  if (state_len < width - 1) return fail(GDN_ERR_SHAPE, "%s: state_len below width - 1", op);
  if (num_slots < 0) return fail(GDN_ERR_SHAPE, "%s: negative num_slots", op);
  return GDN_OK;
}

struct NormIn {
  const void* z;
  int64_t z_rs;
  const void* w;
  float eps;
};

int decode_impl(const char* op, void* out, gdn_dtype out_dt, const void* q, const void* k,
                const void* v, gdn_dtype in_dt, int64_t q_row_stride, int64_t k_row_stride,
                int64_t v_row_stride, const void* alpha, gdn_dtype alpha_dt,
                int64_t alpha_row_stride, const float* dt_bias, const float* ssm_a,
                const void* beta, bool beta_raw, int64_t beta_row_stride, void* state_pool,
                int64_t num_slots, const int32_t* state_idx, int64_t batch, int64_t hk,
                int64_t hv, int64_t dk, int64_t dv, float scale, float l2_eps,
                const NormIn* norm, uint32_t flags, hipStream_t stream) {
  int rc;
  if (batch < 0 || num_slots < 0) return fail(GDN_ERR_SHAPE, "%s: negative batch/num_slots", op);
  if ((rc = check_heads(op, hk, hv, dk, dv))) return rc;
  if ((rc = check_scale(op, scale, l2_eps))) return rc;
  if (!valid_dt(in_dt) || !valid_dt(alpha_dt) || !valid_dt(out_dt))
    return fail(GDN_ERR_DTYPE, "%s: unknown dtype", op);
  if (out_dt != GDN_F32 && out_dt != in_dt)
    return fail(GDN_ERR_DTYPE, "%s: out dtype must be f32 or the input dtype", op);
  const uint32_t known = GDN_L2NORM_QK | GDN_CHECK_SLOTS | GDN_STATE_F16 | GDN_STATE_BF16 |
                         (norm ? (uint32_t)GDN_NORM_SIGMOID : 0u);
  if (flags & ~known) return fail(GDN_ERR_ARG, "%s: unknown flags 0x%x", op, flags);
  if (norm) {
    if (!(norm->eps >= 0.0f) || !isfinite(norm->eps))
      return fail(GDN_ERR_ARG, "%s: norm_eps must be finite and >= 0", op);
    if (dv > gdn::decode_norm_max_dv((int)dk))
      return fail(GDN_ERR_SHAPE, "%s: the fused norm takes dv <= %d at dk = %lld", op,
                  gdn::decode_norm_max_dv((int)dk), (long long)dk);
  }
  const int state_dt = state_dtype(flags);
  if (state_dt < 0) return fail(GDN_ERR_DTYPE, "%s: GDN_STATE_F16 and GDN_STATE_BF16 both set", op);
  if (batch == 0) return ok();
  if (!out || !q || !k || !v || !alpha || !dt_bias || !ssm_a || !beta || !state_pool ||
      !state_idx)
    return fail(GDN_ERR_ARG, "%s: null pointer", op);
  if ((rc = check_qk(op, q, k, in_dt, q_row_stride, k_row_stride, hk, dk))) return rc;
  if (norm) {
    if (!norm->z || !norm->w) return fail(GDN_ERR_ARG, "%s: null pointer", op);
    const size_t eb = (size_t)elem_bytes(in_dt);
    if (!aligned(norm->z, eb) || !aligned(norm->w, eb))
      return fail(GDN_ERR_ARG, "%s: norm_z/norm_w must be aligned to their element size", op);
    if (norm->z_rs < hv * dv)
      return fail(GDN_ERR_SHAPE, "%s: norm_z row stride below hv*dv", op);
  }
  if (v_row_stride < hv * dv || alpha_row_stride < hv || beta_row_stride < hv)
    return fail(GDN_ERR_SHAPE, "%s: v/alpha/beta row stride below its row width", op);
  if (!aligned(state_pool, 16)) return fail(GDN_ERR_ARG, "%s: state pool must be 16-byte aligned", op);
  if (!aligned(alpha, (size_t)elem_bytes(alpha_dt)) ||
      !aligned(beta, beta_raw ? (size_t)elem_bytes(alpha_dt) : 4))
    return fail(GDN_ERR_ARG, "%s: alpha/beta must be aligned to their element size", op);
  if (batch * hv > ((int64_t)1 << 40)) return fail(GDN_ERR_SHAPE, "%s: batch*hv too large", op);
  if (flags & GDN_CHECK_SLOTS) {
    std::vector<int32_t> h;
    if ((rc = fetch_i32(op, state_idx, batch, h, stream))) return rc;
    if ((rc = check_slot_table(op, h, num_slots, true))) return rc;
  }
  gdn::DecodeArgs a{};
  a.out = out; a.out_dt = out_dt; a.q = q; a.k = k; a.v = v; a.in_dt = in_dt;
  a.q_rs = q_row_stride; a.k_rs = k_row_stride; a.v_rs = v_row_stride;
  a.qk_vec = qk_vector_ok(q, k, in_dt, q_row_stride, k_row_stride) ? 1 : 0;
  a.alpha = alpha; a.alpha_dt = alpha_dt; a.alpha_rs = alpha_row_stride;
  a.dt_bias = dt_bias; a.ssm_a = ssm_a; a.beta = beta; a.beta_rs = beta_row_stride;
  a.beta_raw = beta_raw ? 1 : 0;
  a.pool = state_pool; a.state_dt = state_dt; a.num_slots = num_slots; a.idx = state_idx;
  a.batch = batch;
  a.hk = (int)hk; a.hv = (int)hv; a.dk = (int)dk; a.dv = (int)dv;
  a.scale = scale; a.l2_eps = l2_eps; a.l2norm = (flags & GDN_L2NORM_QK) ? 1 : 0;
  if (norm) {
    a.norm_z = norm->z; a.norm_z_rs = norm->z_rs; a.norm_w = norm->w;
    a.norm_eps = norm->eps; a.norm_sigmoid = (flags & GDN_NORM_SIGMOID) ? 1 : 0;
  }
  return hip_status(op, gdn::launch_decode(a, stream));
}

}  // namespace

extern "C" {

int gdn_decode(void* out, gdn_dtype out_dt, const void* q, const void* k, const void* v,
               gdn_dtype in_dt, int64_t q_row_stride, int64_t k_row_stride,
               int64_t v_row_stride, const void* alpha, gdn_dtype alpha_dt,
               int64_t alpha_row_stride, const float* dt_bias, const float* ssm_a,
               const float* beta, int64_t beta_row_stride, void* state_pool,
               int64_t num_slots, const int32_t* state_idx, int64_t batch, int64_t hk,
               int64_t hv, int64_t dk, int64_t dv, float scale, float l2_eps, uint32_t flags,
               hipStream_t stream) {
  return decode_impl("gdn_decode", out, out_dt, q, k, v, in_dt, q_row_stride, k_row_stride,
                     v_row_stride, alpha, alpha_dt, alpha_row_stride, dt_bias, ssm_a, beta,
                     false, beta_row_stride, state_pool, num_slots, state_idx, batch, hk, hv,
                     dk, dv, scale, l2_eps, nullptr, flags, stream);
}

int gdn_decode_packed(void* out, gdn_dtype out_dt, const void* q, const void* k, const void* v,
                      gdn_dtype in_dt, int64_t q_row_stride, int64_t k_row_stride,
                      int64_t v_row_stride, const void* a_raw, const void* b_raw,
                      gdn_dtype ab_dt, int64_t a_row_stride, int64_t b_row_stride,
                      const float* dt_bias, const float* ssm_a, void* state_pool,
                      int64_t num_slots, const int32_t* state_idx, int64_t batch, int64_t hk,
                      int64_t hv, int64_t dk, int64_t dv, float scale, float l2_eps,
                      uint32_t flags, hipStream_t stream) {
  return decode_impl("gdn_decode_packed", out, out_dt, q, k, v, in_dt, q_row_stride,
                     k_row_stride, v_row_stride, a_raw, ab_dt, a_row_stride, dt_bias, ssm_a,
                     b_raw, true, b_row_stride, state_pool, num_slots, state_idx, batch, hk, hv,
                     dk, dv, scale, l2_eps, nullptr, flags, stream);
}

int gdn_decode_gated_norm(void* out, gdn_dtype out_dt, const void* q, const void* k,
                          const void* v, gdn_dtype in_dt, int64_t q_row_stride,
                          int64_t k_row_stride, int64_t v_row_stride, const void* alpha,
                          gdn_dtype alpha_dt, int64_t alpha_row_stride, const float* dt_bias,
                          const float* ssm_a, const float* beta, int64_t beta_row_stride,
                          void* state_pool, int64_t num_slots, const int32_t* state_idx,
                          int64_t batch, int64_t hk, int64_t hv, int64_t dk, int64_t dv,
                          float scale, float l2_eps, const void* norm_z,
                          int64_t norm_z_row_stride, const void* norm_w, float norm_eps,
                          uint32_t flags, hipStream_t stream) {
  const NormIn n{norm_z, norm_z_row_stride, norm_w, norm_eps};
  return decode_impl("gdn_decode_gated_norm", out, out_dt, q, k, v, in_dt, q_row_stride,
                     k_row_stride, v_row_stride, alpha, alpha_dt, alpha_row_stride, dt_bias,
                     ssm_a, beta, false, beta_row_stride, state_pool, num_slots, state_idx,
                     batch, hk, hv, dk, dv, scale, l2_eps, &n, flags, stream);
}

int gdn_rmsnorm_gated(void* out, gdn_dtype out_dt, const void* x, gdn_dtype x_dt,
                      const void* z, int64_t z_row_stride, const void* norm_w, int64_t rows,
                      int64_t hv, int64_t dv, float eps, uint32_t flags, hipStream_t stream) {
  const char* op = "gdn_rmsnorm_gated";
  if (rows < 0 || hv <= 0 || dv <= 0 || hv > (1 << 20) || dv > (1 << 20))
    return fail(GDN_ERR_SHAPE, "%s: rows >= 0, hv and dv in [1, 2^20] required", op);
  if (!valid_dt(x_dt) || !valid_dt(out_dt)) return fail(GDN_ERR_DTYPE, "%s: unknown dtype", op);
  if (out_dt != GDN_F32 && out_dt != x_dt)
    return fail(GDN_ERR_DTYPE, "%s: out dtype must be f32 or the input dtype", op);
  if (flags & ~(uint32_t)GDN_NORM_SIGMOID)
    return fail(GDN_ERR_ARG, "%s: unknown flags 0x%x", op, flags);
  if (!(eps >= 0.0f) || !isfinite(eps))
    return fail(GDN_ERR_ARG, "%s: eps must be finite and >= 0", op);
  if (z_row_stride < hv * dv) return fail(GDN_ERR_SHAPE, "%s: z row stride below hv*dv", op);
  if (rows == 0) return ok();
  if (!out || !x || !z || !norm_w) return fail(GDN_ERR_ARG, "%s: null pointer", op);
  const size_t eb = (size_t)elem_bytes(x_dt);
  if (!aligned(x, eb) || !aligned(z, eb) || !aligned(norm_w, eb) ||
      !aligned(out, (size_t)elem_bytes(out_dt)))
    return fail(GDN_ERR_ARG, "%s: pointers must be aligned to their element size", op);
  if (rows * hv > ((int64_t)1 << 40)) return fail(GDN_ERR_SHAPE, "%s: rows*hv too large", op);
  gdn::NormArgs a{};
  a.out = out; a.out_dt = out_dt; a.x = x; a.x_dt = x_dt; a.z = z; a.z_rs = z_row_stride;
  a.w = norm_w; a.rows = rows; a.hv = (int)hv; a.dv = (int)dv; a.eps = eps;
  a.sigmoid = (flags & GDN_NORM_SIGMOID) ? 1 : 0;
  return hip_status(op, gdn::launch_rmsnorm_gated(a, stream));
}


int gdn_conv1d_fwd(void* out, gdn_dtype out_dt, const void* x, gdn_dtype x_dt,
                   int64_t x_row_stride, const void* weight, const void* bias,
                   void* conv_state, int64_t state_len, int64_t num_slots,
                   const int32_t* state_idx, const int8_t* has_initial_state,
                   const int32_t* cu_seqlens, int64_t num_seqs, int64_t total_tokens,
                   int64_t channels, int64_t width, uint32_t flags, hipStream_t stream) {
  const char* op = "gdn_conv1d_fwd";
  int rc;
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_ERR_SHAPE, "%s: negative size", op);
  if ((rc = conv_common(op, out_dt, x_dt, x_row_stride, state_len, num_slots, channels, width,
                        flags, 0)))
    return rc;
  if (total_tokens >= ((int64_t)1 << 31) * 16)
    return fail(GDN_ERR_SHAPE, "%s: total_tokens too large", op);
  if (num_seqs >= ((int64_t)1 << 31)) return fail(GDN_ERR_SHAPE, "%s: too many sequences", op);
  if (num_seqs == 0) return ok();
  if (width > 1 && !state_idx && num_seqs > num_slots)   // width 1 keeps no state
    return fail(GDN_ERR_SLOT, "%s: %lld sequences but %lld slots", op, (long long)num_seqs,
                (long long)num_slots);
  if (!cu_seqlens || !weight || (width > 1 && !conv_state))
    return fail(GDN_ERR_ARG, "%s: null pointer", op);
  if (total_tokens > 0 && (!out || !x)) return fail(GDN_ERR_ARG, "%s: null pointer", op);
  const size_t ex = (size_t)elem_bytes(x_dt);
  if (!aligned(x, ex) || !aligned(weight, ex) || !aligned(bias, ex) ||
      !aligned(out, (size_t)elem_bytes(out_dt)) ||
      !aligned(conv_state, (size_t)elem_bytes(state_dtype(flags))))
    return fail(GDN_ERR_ARG, "%s: pointers must be aligned to their element size", op);
  if (flags & GDN_CHECK_SLOTS) {
    std::vector<int32_t> h;
    if ((rc = fetch_i32(op, cu_seqlens, num_seqs + 1, h, stream))) return rc;
    if (h[0] != 0 || h[(size_t)num_seqs] != total_tokens)
      return fail(GDN_ERR_SHAPE, "%s: cu_seqlens must run from 0 to total_tokens (%lld)", op,
                  (long long)total_tokens);
    for (int64_t s = 0; s < num_seqs; ++s)
      if (h[(size_t)s + 1] < h[(size_t)s])
        return fail(GDN_ERR_SHAPE, "%s: cu_seqlens decreases at sequence %lld", op,
                    (long long)s);
    if (state_idx && width > 1) {
      if ((rc = fetch_i32(op, state_idx, num_seqs, h, stream))) return rc;
      if ((rc = check_slot_table(op, h, num_slots, false))) return rc;
    }
  }
  gdn::ConvArgs a{};
  a.out = out; a.out_dt = out_dt; a.x = x; a.x_dt = x_dt; a.x_rs = x_row_stride; a.w = weight;
  a.bias = bias; a.state = conv_state; a.state_dt = state_dtype(flags);
  a.state_len = state_len; a.num_slots = num_slots; a.idx = state_idx;
  a.has_init = has_initial_state; a.cu = cu_seqlens; a.n = num_seqs; a.T = total_tokens;
  a.C = channels; a.K = (int)width; a.silu = (flags & GDN_CONV_SILU) ? 1 : 0;
  return hip_status(op, gdn::launch_conv_fwd(a, stream));
}

int gdn_conv1d_update(void* out, gdn_dtype out_dt, const void* x, gdn_dtype x_dt,
                      int64_t x_row_stride, const void* weight, const void* bias,
                      void* conv_state, int64_t state_len, int64_t num_slots,
                      const int32_t* state_idx, int64_t batch, int64_t channels, int64_t width,
                      uint32_t flags, hipStream_t stream) {
  const char* op = "gdn_conv1d_update";
  int rc;
  if (batch < 0) return fail(GDN_ERR_SHAPE, "%s: negative batch", op);
  if ((rc = conv_common(op, out_dt, x_dt, x_row_stride, state_len, num_slots, channels, width,
                        flags, 0)))
    return rc;
  if (batch >= ((int64_t)1 << 31)) return fail(GDN_ERR_SHAPE, "%s: batch too large", op);
  if (batch == 0) return ok();
  if (width > 1 && !state_idx && batch > num_slots)   // width 1 keeps no state
    return fail(GDN_ERR_SLOT, "%s: %lld rows but %lld slots", op, (long long)batch,
                (long long)num_slots);
  if (!out || !x || !weight || (width > 1 && !conv_state))
    return fail(GDN_ERR_ARG, "%s: null pointer", op);
  const size_t ex = (size_t)elem_bytes(x_dt);
  if (!aligned(x, ex) || !aligned(weight, ex) || !aligned(bias, ex) ||
      !aligned(out, (size_t)elem_bytes(out_dt)) ||
      !aligned(conv_state, (size_t)elem_bytes(state_dtype(flags))))
    return fail(GDN_ERR_ARG, "%s: pointers must be aligned to their element size", op);
  if ((flags & GDN_CHECK_SLOTS) && state_idx && width > 1) {
    std::vector<int32_t> h;
    if ((rc = fetch_i32(op, state_idx, batch, h, stream))) return rc;
    if ((rc = check_slot_table(op, h, num_slots, true))) return rc;
  }
  gdn::ConvArgs a{};
  a.out = out; a.out_dt = out_dt; a.x = x; a.x_dt = x_dt; a.x_rs = x_row_stride; a.w = weight;
  a.bias = bias; a.state = conv_state; a.state_dt = state_dtype(flags);
  a.state_len = state_len; a.num_slots = num_slots; a.idx = state_idx; a.n = batch;
  a.C = channels; a.K = (int)width; a.silu = (flags & GDN_CONV_SILU) ? 1 : 0;
  return hip_status(op, gdn::launch_conv_update(a, stream));
}

static bool use_chunked(int64_t hk, int64_t hv, int64_t dk, int64_t dv, int in_dt, int out_dt,
                        uint32_t flags) {
  (void)hk;
  return !(flags & GDN_PREFILL_SEQUENTIAL) && gdn::chunked_supported(in_dt, out_dt, hv, (int)dk, (int)dv);
}

size_t gdn_prefill_varlen_workspace_size(int64_t total_tokens, int64_t num_seqs, int64_t hk,
                                         int64_t hv, int64_t dk, int64_t dv, gdn_dtype in_dt,
                                         uint32_t flags) {
  if (total_tokens <= 0 || num_seqs <= 0 || hk <= 0 || hv <= 0 || dk <= 0 || dv <= 0) return 0;
  if (!use_chunked(hk, hv, dk, dv, in_dt, in_dt, flags)) return 0;
  return gdn::chunked_workspace_bytes(total_tokens, num_seqs, (int)hv, (int)dk, (int)dv);
}

}  // extern "C"

namespace {

// gdn_prefill_varlen, its variant with the caller's second stream (aux, for
// the split schedule; null: the caller's stream alone) and its
// allocation-free variant (which passes the library's per-device scratch as
// the workspace).
// Where a prefill takes g and beta from: g materialised (f32), or formed in
// the kernels from alpha (alpha_dt) with dt_bias and ssm_a; beta as f32
// post-sigmoid values, or (beta_raw) the raw b in alpha_dt.
struct GateIn {
  const float* g;
  int64_t g_rs;
  const void* alpha;
  gdn_dtype alpha_dt;
  int64_t alpha_rs;
  const float* dt_bias;
  const float* ssm_a;
  const void* beta;
  int64_t beta_rs;
  bool beta_raw;
};

int prefill_impl(const char* op, void* out, gdn_dtype out_dt, const void* q, const void* k,
                 const void* v, gdn_dtype in_dt, int64_t q_row_stride, int64_t k_row_stride,
                 int64_t v_row_stride, const GateIn& gt, void* state_pool, int64_t num_slots,
                 const int32_t* state_idx, const int8_t* has_initial_state,
                 const int32_t* cu_seqlens, int64_t num_seqs, int64_t total_tokens, int64_t hk,
                 int64_t hv, int64_t dk, int64_t dv, float scale, float l2_eps, uint32_t flags,
                 void* workspace, size_t workspace_bytes, hipStream_t stream, hipStream_t aux) {
  int rc;
  if (num_seqs < 0 || total_tokens < 0 || num_slots < 0)
    return fail(GDN_ERR_SHAPE, "%s: negative size", op);
  if ((rc = check_heads(op, hk, hv, dk, dv))) return rc;
  if ((rc = check_scale(op, scale, l2_eps))) return rc;
  if (!valid_dt(in_dt) || !valid_dt(out_dt)) return fail(GDN_ERR_DTYPE, "%s: unknown dtype", op);
  if (out_dt != GDN_F32 && out_dt != in_dt)
    return fail(GDN_ERR_DTYPE, "%s: out dtype must be f32 or the input dtype", op);
  if (flags & ~(uint32_t)(GDN_L2NORM_QK | GDN_CHECK_SLOTS | GDN_PREFILL_SEQUENTIAL |
                          GDN_STATE_F16 | GDN_STATE_BF16 |
                          (gt.beta_raw ? (uint32_t)GDN_BETA_ROUNDED : 0u)))
    return fail(GDN_ERR_ARG, "%s: unknown flags 0x%x", op, flags);
  if (gt.alpha && !valid_dt(gt.alpha_dt)) return fail(GDN_ERR_DTYPE, "%s: unknown dtype", op);
  const int state_dt = state_dtype(flags);
  if (state_dt < 0) return fail(GDN_ERR_DTYPE, "%s: GDN_STATE_F16 and GDN_STATE_BF16 both set", op);
  if (num_seqs == 0) return ok();
  if (!state_pool || !cu_seqlens) return fail(GDN_ERR_ARG, "%s: null pointer", op);
  if (!state_idx && num_seqs > num_slots)
    return fail(GDN_ERR_SLOT, "%s: %lld sequences but %lld slots", op, (long long)num_seqs,
                (long long)num_slots);
  if (!aligned(state_pool, 16)) return fail(GDN_ERR_ARG, "%s: state pool must be 16-byte aligned", op);
  if (total_tokens > 0) {
    if (!out || !q || !k || !v || !gt.beta || (gt.alpha ? !gt.dt_bias || !gt.ssm_a : !gt.g))
      return fail(GDN_ERR_ARG, "%s: null pointer", op);
    if ((rc = check_qk(op, q, k, in_dt, q_row_stride, k_row_stride, hk, dk))) return rc;
    if (v_row_stride < hv * dv || (gt.alpha ? gt.alpha_rs : gt.g_rs) < hv || gt.beta_rs < hv)
      return fail(GDN_ERR_SHAPE, "%s: v/gate/beta row stride below its row width", op);
    const size_t ab = gt.alpha ? (size_t)elem_bytes(gt.alpha_dt) : 4;
    if ((gt.alpha && !aligned(gt.alpha, ab)) || !aligned(gt.beta, gt.beta_raw ? ab : 4))
      return fail(GDN_ERR_ARG, "%s: gate inputs must be aligned to their element size", op);
  }
  if (flags & GDN_CHECK_SLOTS) {
    std::vector<int32_t> h;
    if ((rc = fetch_i32(op, cu_seqlens, num_seqs + 1, h, stream))) return rc;
    if (h[0] != 0 || h[(size_t)num_seqs] != total_tokens)
      return fail(GDN_ERR_SHAPE, "%s: cu_seqlens must run from 0 to total_tokens (%lld)", op,
                  (long long)total_tokens);
    for (int64_t s = 0; s < num_seqs; ++s)
      if (h[(size_t)s + 1] < h[(size_t)s])
        return fail(GDN_ERR_SHAPE, "%s: cu_seqlens decreases at sequence %lld", op,
                    (long long)s);
    if (state_idx) {
      if ((rc = fetch_i32(op, state_idx, num_seqs, h, stream))) return rc;
      if ((rc = check_slot_table(op, h, num_slots, false))) return rc;
    }
  }
  gdn::PrefillArgs a{};
  a.out = out; a.out_dt = out_dt; a.q = q; a.k = k; a.v = v; a.in_dt = in_dt;
  a.q_rs = q_row_stride; a.k_rs = k_row_stride; a.v_rs = v_row_stride;
  a.qk_vec = qk_vector_ok(q, k, in_dt, q_row_stride, k_row_stride) ? 1 : 0;
  a.g = gt.g; a.g_rs = gt.g_rs; a.beta = gt.beta; a.beta_rs = gt.beta_rs;
  a.alpha = gt.alpha; a.alpha_dt = gt.alpha_dt; a.alpha_rs = gt.alpha_rs;
  a.dt_bias = gt.dt_bias; a.ssm_a = gt.ssm_a; a.beta_raw = gt.beta_raw ? 1 : 0;
  a.round_beta = (flags & GDN_BETA_ROUNDED) ? 1 : 0;
  a.pool = state_pool; a.state_dt = state_dt; a.num_slots = num_slots; a.idx = state_idx;
  a.has_init = has_initial_state; a.cu = cu_seqlens; a.num_seqs = num_seqs;
  a.total_tokens = total_tokens;
  a.hk = (int)hk; a.hv = (int)hv; a.dk = (int)dk; a.dv = (int)dv;
  a.scale = scale; a.l2_eps = l2_eps; a.l2norm = (flags & GDN_L2NORM_QK) ? 1 : 0;
  if (use_chunked(hk, hv, dk, dv, in_dt, out_dt, flags) && total_tokens > 0 &&
      gdn::chunked_layout_ok(q, k, v, q_row_stride, k_row_stride, v_row_stride)) {
    const size_t need = gdn::chunked_workspace_bytes(total_tokens, num_seqs, (int)hv, (int)dk,
                                                     (int)dv);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(GDN_ERR_ARG, "%s: workspace of %zu bytes required, got %zu", op, need,
                  workspace_bytes);
    if (need > 0 && !aligned(workspace, 256))
      return fail(GDN_ERR_ARG, "%s: workspace must be 256-byte aligned", op);
    return hip_status(op, gdn::launch_prefill_chunked(a, workspace, workspace_bytes, stream, aux));
  }
  return hip_status(op, gdn::launch_prefill_sequential(a, stream));
}


// Scratch of gdn_prefill_varlen_noalloc: one copy of this array per device,
// held until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's scratch address (resolved on the first call on that
// device, with it current), or nullptr with the error message set.
void* device_scratch(const char* op) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
    fail(GDN_ERR_HIP, "%s: no current device (or device index %d too large)", op, dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fail(GDN_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed: %s", op, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int gdn_prefill_varlen(void* out, gdn_dtype out_dt, const void* q, const void* k, const void* v,
                       gdn_dtype in_dt, int64_t q_row_stride, int64_t k_row_stride,
                       int64_t v_row_stride, const float* g, int64_t g_row_stride,
                       const float* beta, int64_t beta_row_stride, void* state_pool,
                       int64_t num_slots, const int32_t* state_idx,
                       const int8_t* has_initial_state, const int32_t* cu_seqlens,
                       int64_t num_seqs, int64_t total_tokens, int64_t hk, int64_t hv,
                       int64_t dk, int64_t dv, float scale, float l2_eps, uint32_t flags,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const GateIn gt{g, g_row_stride, nullptr, GDN_F32, 0, nullptr, nullptr, beta, beta_row_stride,
                  false};
  return prefill_impl("gdn_prefill_varlen", out, out_dt, q, k, v, in_dt, q_row_stride,
                      k_row_stride, v_row_stride, gt, state_pool, num_slots, state_idx,
                      has_initial_state, cu_seqlens, num_seqs, total_tokens, hk, hv, dk, dv,
                      scale, l2_eps, flags, workspace, workspace_bytes, stream, nullptr);
}

int gdn_prefill_varlen_aux(void* out, gdn_dtype out_dt, const void* q, const void* k,
                           const void* v, gdn_dtype in_dt, int64_t q_row_stride,
                           int64_t k_row_stride, int64_t v_row_stride, const float* g,
                           int64_t g_row_stride, const float* beta, int64_t beta_row_stride,
                           void* state_pool, int64_t num_slots, const int32_t* state_idx,
                           const int8_t* has_initial_state, const int32_t* cu_seqlens,
                           int64_t num_seqs, int64_t total_tokens, int64_t hk, int64_t hv,
                           int64_t dk, int64_t dv, float scale, float l2_eps, uint32_t flags,
                           void* workspace, size_t workspace_bytes, hipStream_t stream,
                           hipStream_t aux_stream) {
  const GateIn gt{g, g_row_stride, nullptr, GDN_F32, 0, nullptr, nullptr, beta, beta_row_stride,
                  false};
  return prefill_impl("gdn_prefill_varlen_aux", out, out_dt, q, k, v, in_dt, q_row_stride,
                      k_row_stride, v_row_stride, gt, state_pool, num_slots, state_idx,
                      has_initial_state, cu_seqlens, num_seqs, total_tokens, hk, hv, dk, dv,
                      scale, l2_eps, flags, workspace, workspace_bytes, stream, aux_stream);
}

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
                             hipStream_t aux_stream) {
  const GateIn gt{nullptr, 0, alpha, alpha_dt, alpha_row_stride, dt_bias, ssm_a, beta,
                  beta_row_stride, false};
  return prefill_impl("gdn_prefill_varlen_gated", out, out_dt, q, k, v, in_dt, q_row_stride,
                      k_row_stride, v_row_stride, gt, state_pool, num_slots, state_idx,
                      has_initial_state, cu_seqlens, num_seqs, total_tokens, hk, hv, dk, dv,
                      scale, l2_eps, flags, workspace, workspace_bytes, stream, aux_stream);
}

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
                                  hipStream_t stream, hipStream_t aux_stream) {
  const char* op = "gdn_prefill_varlen_gated_norm";
  // the norm's arguments are checked before the prefill enqueues anything
  if (!valid_dt(in_dt) || !valid_dt(out_dt)) return fail(GDN_ERR_DTYPE, "%s: unknown dtype", op);
  if (out_dt != in_dt)
    return fail(GDN_ERR_DTYPE, "%s: out dtype must be the input dtype (norm_z and norm_w share it)",
                op);
  if (!(norm_eps >= 0.0f) || !isfinite(norm_eps))
    return fail(GDN_ERR_ARG, "%s: norm_eps must be finite and >= 0", op);
  const bool rows = num_seqs > 0 && total_tokens > 0;
  if (rows) {
    if (hv <= 0 || dv <= 0 || hv > (1 << 20) || dv > (1 << 20))
      return fail(GDN_ERR_SHAPE, "%s: hv and dv in [1, 2^20] required", op);
    if (norm_z_row_stride < hv * dv)
      return fail(GDN_ERR_SHAPE, "%s: norm_z row stride below hv*dv", op);
    if (!norm_z || !norm_w) return fail(GDN_ERR_ARG, "%s: null pointer", op);
    const size_t eb = (size_t)elem_bytes(in_dt);
    if (!aligned(norm_z, eb) || !aligned(norm_w, eb))
      return fail(GDN_ERR_ARG, "%s: norm_z/norm_w must be aligned to their element size", op);
    if (total_tokens * hv > ((int64_t)1 << 40))
      return fail(GDN_ERR_SHAPE, "%s: total_tokens*hv too large", op);
  }
  const GateIn gt{nullptr, 0, alpha, alpha_dt, alpha_row_stride, dt_bias, ssm_a, beta,
                  beta_row_stride, false};
  const int rc = prefill_impl(op, out, out_dt, q, k, v, in_dt, q_row_stride, k_row_stride,
                              v_row_stride, gt, state_pool, num_slots, state_idx,
                              has_initial_state, cu_seqlens, num_seqs, total_tokens, hk, hv, dk,
                              dv, scale, l2_eps, flags & ~(uint32_t)GDN_NORM_SIGMOID, workspace,
                              workspace_bytes, stream, aux_stream);
  if (rc != GDN_OK || !rows) return rc;
  // the norm in place over out, behind every walk (the second stream has
  // joined `stream` by now); each lane reads its elements before it writes them
  gdn::NormArgs a{};
  a.out = out; a.out_dt = out_dt; a.x = out; a.x_dt = out_dt; a.z = norm_z;
  a.z_rs = norm_z_row_stride; a.w = norm_w; a.rows = total_tokens; a.hv = (int)hv;
  a.dv = (int)dv; a.eps = norm_eps; a.sigmoid = (flags & GDN_NORM_SIGMOID) ? 1 : 0;
  return hip_status(op, gdn::launch_rmsnorm_gated(a, stream));
}

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
                              hipStream_t aux_stream) {
  const GateIn gt{nullptr, 0, a_raw, ab_dt, a_row_stride, dt_bias, ssm_a, b_raw, b_row_stride,
                  true};
  return prefill_impl("gdn_prefill_varlen_packed", out, out_dt, q, k, v, in_dt, q_row_stride,
                      k_row_stride, v_row_stride, gt, state_pool, num_slots, state_idx,
                      has_initial_state, cu_seqlens, num_seqs, total_tokens, hk, hv, dk, dv,
                      scale, l2_eps, flags, workspace, workspace_bytes, stream, aux_stream);
}

int gdn_prefill_varlen_noalloc(void* out, gdn_dtype out_dt, const void* q, const void* k,
                               const void* v, gdn_dtype in_dt, int64_t q_row_stride,
                               int64_t k_row_stride, int64_t v_row_stride, const float* g,
                               int64_t g_row_stride, const float* beta,
                               int64_t beta_row_stride, void* state_pool, int64_t num_slots,
                               const int32_t* state_idx, const int8_t* has_initial_state,
                               const int32_t* cu_seqlens, int64_t num_seqs,
                               int64_t total_tokens, int64_t hk, int64_t hv, int64_t dk,
                               int64_t dv, float scale, float l2_eps, uint32_t flags,
                               hipStream_t stream) {
  const char* op = "gdn_prefill_varlen_noalloc";
  const size_t need = gdn_prefill_varlen_workspace_size(total_tokens, num_seqs, hk, hv, dk, dv,
                                                        in_dt, flags);
  if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
    return fail(GDN_ERR_SHAPE,
                "%s: these sizes need %zu bytes of scratch, more than the %zu this entry "
                "point holds per device; use gdn_prefill_varlen with a workspace",
                op, need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0 && !(ws = device_scratch(op))) return GDN_ERR_HIP;
  const GateIn gt{g, g_row_stride, nullptr, GDN_F32, 0, nullptr, nullptr, beta, beta_row_stride,
                  false};
  return prefill_impl(op, out, out_dt, q, k, v, in_dt, q_row_stride, k_row_stride,
                      v_row_stride, gt, state_pool, num_slots, state_idx, has_initial_state,
                      cu_seqlens, num_seqs, total_tokens, hk, hv, dk, dv, scale, l2_eps, flags,
                      ws, ws ? (size_t)GDN_NOALLOC_SCRATCH_BYTES : 0, stream, nullptr);
}

}  // extern "C"
