/*
 * gdn_oracle.c -- plain, slow CPU reference for the Gated DeltaNet hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the GPU library and neither one includes the other.
 *
 * Everything is computed in double precision from the exact input bytes the GPU
 * reads (f32, IEEE-754 binary16 or bfloat16, decoded here by this file's own
 * routines), token by token, with no blocking, fusion or reassociation beyond
 * what the definitions below state.  Results are returned unrounded in f64.
 *
 * Sources (the web pages this method is defined on):
 *  - Winery-Strata, src/kernels/elementwise_parity.cpp, "1. gdn_gate" block:
 *    the gate g = softplus(alpha + dt_bias) * ssm_a, softplus returning x when
 *    x > 20 and log1p(exp(x)) otherwise, computed in double.
 *  - vllm.cpp, tests/vt/test_ops_gdn.cpp:
 *      "gdn decode: hand-computed single step" (the per-token recurrence:
 *       decay, S@k, v', rank-1 update, output from the updated state; state
 *       rows index v, columns index k);
 *      "gdn prefill: hand-computed 3-token recurrence table" and the varlen
 *       test (cu_seqlens segments, per-sequence state read then overwritten);
 *      "gdn decode + conv update: indexed in-place == compact reference"
 *       (state addressed through per-sequence slot indices);
 *      PackedDecodeReference (q/k L2-norm with eps inside the square root,
 *       q scaled after normalising, GQA head hk = hv / (Hv/Hk), slot < 0 gives
 *       a zero output row and leaves the state alone, duplicate or
 *       out-of-range live slots are errors);
 *      "l2norm: plain sum of squares over the last dim";
 *      "rmsnorm_gated: norm-then-gate, silu and sigmoid activations" and the
 *       rank-3 padded-row gate case (the gated RMSNorm after the recurrence);
 *      "gdn_post_conv fused == composed" and the packed in_proj_ba case (the
 *       front-end: conv output split into q, k, v, q/k normalised, g and
 *       beta = sigmoid(b) from a and b views of one merged row);
 *      PackedDecodeReference's beta, sigmoid(b) rounded through b's dtype;
 *      the causal_conv1d_fwd / causal_conv1d_update cases (depthwise causal
 *       conv with a K-1 state per channel, bias, silu, varlen with
 *       has_initial_state, the T < K-1 write-back, indexed and widened caches).
 *
 * Parity pins live in tests/test_oracle_pins.py (the pages' worked values and
 * the invariants listed there).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_F16 1
#define OR_BF16 2
#define OR_F64 3 /* oracle-internal: an array of doubles (e.g. an f64 output) */

#define OR_OK 0
#define OR_ERR_ARG -1
#define OR_ERR_SHAPE -3
#define OR_ERR_SLOT -4

/* ------------------------------------------------------------------------
 * Storage decoders, from the format definitions.
 *  binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits;
 *            exponent 0 = subnormal (fraction * 2^-24), 31 = inf/NaN.
 *  bfloat16: the top 16 bits of an IEEE-754 binary32.
 * ------------------------------------------------------------------------ */
static double half_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1f;
  const int f = h & 0x3ff;
  double mag;
  if (e == 0) {
    mag = ldexp((double)f, -24);
  } else if (e == 31) {
    mag = f ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(1024 + f), e - 25);
  }
  return sign ? -mag : mag;
}

static double bf16_to_double(uint16_t b) {
  uint32_t bits = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

static double load_elem(const void* base, int dt, int64_t off) {
  switch (dt) {
    case OR_F32: return (double)((const float*)base)[off];
    case OR_F16: return half_to_double(((const uint16_t*)base)[off]);
    case OR_BF16: return bf16_to_double(((const uint16_t*)base)[off]);
    case OR_F64: return ((const double*)base)[off];
    default: return NAN;
  }
}

/* exported so the tests can pin the decoders against the format definitions */
double oracle_decode_value(const void* base, int dt, int64_t off) {
  return load_elem(base, dt, off);
}

/* ------------------------------------------------------------------------
 * Gate (Winery-Strata elementwise_parity.cpp, gdn_gate fixture):
 *   x  = alpha + dt_bias[h]
 *   sp = x > 20 ? x : log1p(exp(x))
 *   g  = sp * ssm_a[h]           (ssm_a = -exp(A_log) < 0 is given)
 * alpha is [rows, hv] with a row stride in elements.  g is [rows, hv] f64.
 * ------------------------------------------------------------------------ */
static double softplus_branch(double x) { return x > 20.0 ? x : log1p(exp(x)); }

void oracle_softplus(const double* x, double* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = softplus_branch(x[i]);
}

int oracle_gate(int64_t rows, int64_t hv, const void* alpha, int alpha_dt,
                int64_t alpha_row_stride, const float* dt_bias, const float* ssm_a,
                double* g) {
  if (rows < 0 || hv <= 0 || alpha_row_stride < hv) return OR_ERR_SHAPE;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t h = 0; h < hv; ++h) {
      const double x = load_elem(alpha, alpha_dt, r * alpha_row_stride + h) + (double)dt_bias[h];
      g[r * hv + h] = softplus_branch(x) * (double)ssm_a[h];
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------------
 * L2 norm over the last dim (vllm.cpp "l2norm: plain sum of squares"):
 *   y = x / sqrt(sum_d x_d^2 + eps)
 * ------------------------------------------------------------------------ */
static void l2_normalize(double* x, int64_t d, double eps) {
  double ss = 0.0;
  for (int64_t i = 0; i < d; ++i) ss += x[i] * x[i];
  const double inv = 1.0 / sqrt(ss + eps);
  for (int64_t i = 0; i < d; ++i) x[i] *= inv;
}

void oracle_l2norm(const double* x, double* y, int64_t rows, int64_t d, double eps) {
  for (int64_t r = 0; r < rows; ++r) {
    memcpy(y + r * d, x + r * d, (size_t)d * sizeof(double));
    l2_normalize(y + r * d, d, eps);
  }
}

/* ------------------------------------------------------------------------
 * One token of the gated delta rule on one head (vllm.cpp, "gdn decode:
 * hand-computed single step").  S is [dv][dk], rows index v, columns index k.
 *   S  *= exp(g)
 *   sk  = S @ k
 *   v'  = beta * (v - sk)
 *   S  += v' (outer) k
 *   o   = S @ q            (q already normalised and scaled; updated S)
 * ------------------------------------------------------------------------ */
static void recurrence_step(double* S, int64_t dv, int64_t dk, const double* k,
                            const double* q, const double* v, double g, double beta,
                            double* o, double* work /* [dv] */) {
  const double decay = exp(g);
  for (int64_t i = 0; i < dv * dk; ++i) S[i] *= decay;
  for (int64_t i = 0; i < dv; ++i) {
    double sk = 0.0;
    for (int64_t j = 0; j < dk; ++j) sk += S[i * dk + j] * k[j];
    work[i] = beta * (v[i] - sk);
  }
  for (int64_t i = 0; i < dv; ++i)
    for (int64_t j = 0; j < dk; ++j) S[i * dk + j] += work[i] * k[j];
  for (int64_t i = 0; i < dv; ++i) {
    double acc = 0.0;
    for (int64_t j = 0; j < dk; ++j) acc += S[i * dk + j] * q[j];
    o[i] = acc;
  }
}

/* Load token `row`'s q and k head `hk` and v head `hv`, normalise and scale. */
static void load_qkv(const void* q, const void* k, const void* v, int in_dt, int64_t q_rs,
                     int64_t k_rs, int64_t v_rs, int64_t row, int64_t hk, int64_t hv,
                     int64_t dk, int64_t dv, int l2norm, double l2_eps, double scale,
                     double* qd, double* kd, double* vd) {
  for (int64_t j = 0; j < dk; ++j) {
    qd[j] = load_elem(q, in_dt, row * q_rs + hk * dk + j);
    kd[j] = load_elem(k, in_dt, row * k_rs + hk * dk + j);
  }
  for (int64_t i = 0; i < dv; ++i) vd[i] = load_elem(v, in_dt, row * v_rs + hv * dv + i);
  if (l2norm) {
    l2_normalize(qd, dk, l2_eps);
    l2_normalize(kd, dk, l2_eps);
  }
  for (int64_t j = 0; j < dk; ++j) qd[j] *= scale;
}

static int check_common(int64_t hk, int64_t hv, int64_t dk, int64_t dv, double scale) {
  if (hk <= 0 || hv <= 0 || dk <= 0 || dv <= 0) return OR_ERR_SHAPE;
  if (hv % hk != 0) return OR_ERR_SHAPE;
  if (!(scale > 0.0) || !isfinite(scale)) return OR_ERR_ARG;
  return OR_OK;
}

/* live slots must be in range and distinct (PackedDecodeReference's caller
   rejects duplicate and out-of-range live slots) */
static int check_slots(const int32_t* idx, int64_t n, int64_t num_slots, int allow_null) {
  char* seen = (char*)calloc((size_t)(num_slots > 0 ? num_slots : 1), 1);
  if (!seen) return OR_ERR_ARG;
  int rc = OR_OK;
  for (int64_t b = 0; b < n; ++b) {
    const int32_t s = idx[b];
    if (s < 0) {
      if (!allow_null) { rc = OR_ERR_SLOT; break; }
      continue;
    }
    if (s >= num_slots || seen[s]) { rc = OR_ERR_SLOT; break; }
    seen[s] = 1;
  }
  free(seen);
  return rc;
}

/* ------------------------------------------------------------------------
 * Independent units on several host threads.  The recurrence never mixes
 * sequences or v-heads, so each (row or sequence, v-head) unit is computed
 * alone, in the order written above, by whichever thread takes it; the
 * arithmetic of a unit does not depend on the thread count.  Every thread
 * owns its own scratch vectors.
 * ------------------------------------------------------------------------ */
static int g_threads = 1;

void oracle_set_threads(int n) { g_threads = n < 1 ? 1 : (n > 256 ? 256 : n); }
int oracle_get_threads(void) { return g_threads; }

typedef void (*unit_fn)(const void* ctx, int64_t unit, double* scratch);

struct unit_job {
  unit_fn fn;
  const void* ctx;
  int64_t n_units;
  int64_t next; /* taken with an atomic add */
  size_t scratch_len;
  int failed;
};

static void* unit_worker(void* arg) {
  struct unit_job* job = (struct unit_job*)arg;
  double* scratch = (double*)malloc(job->scratch_len * sizeof(double));
  if (!scratch) {
    __atomic_store_n(&job->failed, 1, __ATOMIC_RELAXED);
    return NULL;
  }
  for (;;) {
    const int64_t u = __atomic_fetch_add(&job->next, 1, __ATOMIC_RELAXED);
    if (u >= job->n_units) break;
    job->fn(job->ctx, u, scratch);
  }
  free(scratch);
  return NULL;
}

static int run_units(unit_fn fn, const void* ctx, int64_t n_units, size_t scratch_len) {
  struct unit_job job = {fn, ctx, n_units, 0, scratch_len, 0};
  int nt = g_threads;
  if ((int64_t)nt > n_units) nt = n_units > 0 ? (int)n_units : 1;
  pthread_t tids[256];
  int started = 0;
  for (int i = 1; i < nt; ++i) {
    if (pthread_create(&tids[started], NULL, unit_worker, &job) != 0) break;
    ++started;
  }
  unit_worker(&job); /* the calling thread works too */
  for (int i = 0; i < started; ++i) pthread_join(tids[i], NULL);
  return job.failed ? OR_ERR_ARG : OR_OK;
}

/* ------------------------------------------------------------------------
 * Decode: one token for each of `batch` sequences.  Sequence b's state is
 * pool[idx[b]] ([hv][dv][dk], read only here, stored as f32, f16 or bf16 per
 * state_dt and widened exactly to f64); idx[b] < 0 marks a padded
 * row whose output is zero and whose state is not touched.
 * g is [batch, hv] (from oracle_gate), beta is [batch, hv] f32 with a row stride.
 * Outputs: out [batch, hv, dv] f64; state_out [batch, hv, dv, dk] f64 holding
 * the updated state of each live row (rows with idx < 0 are left as given).
 * head_mask [hv] (NULL = all heads) restricts the work to the marked v-heads;
 * entries of other heads are left as given.
 * ------------------------------------------------------------------------ */
struct decode_ctx {
  int64_t hk, hv, dk, dv, ratio;
  const void *q, *k, *v;
  int in_dt;
  int64_t q_rs, k_rs, v_rs;
  const double* g;
  const float* beta;
  int64_t beta_rs;
  const void* pool;
  int state_dt;
  const int32_t* idx;
  double scale, l2_eps;
  int l2norm;
  const uint8_t* head_mask;
  double *out, *state_out;
};

/* unit = (row b, v-head h) */
static void decode_unit(const void* cp, int64_t u, double* scratch) {
  const struct decode_ctx* c = (const struct decode_ctx*)cp;
  const int64_t b = u / c->hv, h = u % c->hv;
  if (c->head_mask && !c->head_mask[h]) return;
  const int64_t dk = c->dk, dv = c->dv, head_elems = dv * dk;
  double *qd = scratch, *kd = qd + dk, *vd = kd + dk, *work = vd + dv;
  double* o = c->out + (b * c->hv + h) * dv;
  const int32_t slot = c->idx[b];
  if (slot < 0) {
    for (int64_t i = 0; i < dv; ++i) o[i] = 0.0;
    return;
  }
  load_qkv(c->q, c->k, c->v, c->in_dt, c->q_rs, c->k_rs, c->v_rs, b, h / c->ratio, h, dk, dv,
           c->l2norm, c->l2_eps, c->scale, qd, kd, vd);
  double* S = c->state_out + (b * c->hv + h) * head_elems;
  const int64_t s0 = ((int64_t)slot * c->hv + h) * head_elems;
  for (int64_t e = 0; e < head_elems; ++e) S[e] = load_elem(c->pool, c->state_dt, s0 + e);
  recurrence_step(S, dv, dk, kd, qd, vd, c->g[b * c->hv + h],
                  (double)c->beta[b * c->beta_rs + h], o, work);
}

int oracle_decode(int64_t batch, int64_t hk, int64_t hv, int64_t dk, int64_t dv,
                  const void* q, const void* k, const void* v, int in_dt, int64_t q_rs,
                  int64_t k_rs, int64_t v_rs, const double* g, const float* beta,
                  int64_t beta_rs, const void* pool, int state_dt, int64_t num_slots,
                  const int32_t* idx, double scale, double l2_eps, int l2norm,
                  const uint8_t* head_mask,
                  double* out, double* state_out) {
  int rc = check_common(hk, hv, dk, dv, scale);
  if (rc) return rc;
  if (state_dt != OR_F32 && state_dt != OR_F16 && state_dt != OR_BF16) return OR_ERR_ARG;
  rc = check_slots(idx, batch, num_slots, 1);
  if (rc) return rc;
  const struct decode_ctx c = {hk, hv, dk, dv, hv / hk, q, k, v, in_dt, q_rs, k_rs, v_rs,
                               g, beta, beta_rs, pool, state_dt, idx, scale, l2_eps, l2norm,
                               head_mask, out, state_out};
  return run_units(decode_unit, &c, batch * hv, (size_t)(2 * dk + 2 * dv));
}

/* ------------------------------------------------------------------------
 * Varlen prefill.  Sequence s covers tokens [cu[s], cu[s+1]).  Its state starts
 * as pool[idx[s]] when has_init[s] != 0 (has_init == NULL: all 1), else as
 * zeros (the slot is then never read); idx == NULL means slot s.  The
 * recurrence runs over the sequence's tokens in order and the final state of
 * each sequence is returned in state_out [num_seqs, hv, dv, dk] f64.
 * g, beta: [T, hv] (g f64 from oracle_gate; beta f32 with a row stride).
 * out: [T, hv, dv] f64.  head_mask as for oracle_decode.
 * ------------------------------------------------------------------------ */
struct prefill_ctx {
  const int32_t* cu;
  int64_t hk, hv, dk, dv, ratio;
  const void *q, *k, *v;
  int in_dt;
  int64_t q_rs, k_rs, v_rs;
  const double* g;
  const float* beta;
  int64_t beta_rs;
  const void* pool;
  int state_dt;
  const int32_t* idx;
  const int8_t* has_init;
  double scale, l2_eps;
  int l2norm;
  const uint8_t* head_mask;
  double *out, *state_out;
};

/* unit = (sequence s, v-head h): the whole token loop of that head */
static void prefill_unit(const void* cp, int64_t u, double* scratch) {
  const struct prefill_ctx* c = (const struct prefill_ctx*)cp;
  const int64_t s = u / c->hv, h = u % c->hv;
  if (c->head_mask && !c->head_mask[h]) return;
  const int64_t dk = c->dk, dv = c->dv, head_elems = dv * dk;
  double *qd = scratch, *kd = qd + dk, *vd = kd + dk, *work = vd + dv;
  const int64_t slot = c->idx ? c->idx[s] : s;
  const int init = c->has_init ? c->has_init[s] != 0 : 1;
  double* S = c->state_out + (s * c->hv + h) * head_elems;
  const int64_t s0 = (slot * c->hv + h) * head_elems;
  for (int64_t e = 0; e < head_elems; ++e)
    S[e] = init ? load_elem(c->pool, c->state_dt, s0 + e) : 0.0;
  const int64_t hkh = h / c->ratio;
  for (int64_t t = c->cu[s]; t < c->cu[s + 1]; ++t) {
    load_qkv(c->q, c->k, c->v, c->in_dt, c->q_rs, c->k_rs, c->v_rs, t, hkh, h, dk, dv,
             c->l2norm, c->l2_eps, c->scale, qd, kd, vd);
    recurrence_step(S, dv, dk, kd, qd, vd, c->g[t * c->hv + h],
                    (double)c->beta[t * c->beta_rs + h], c->out + (t * c->hv + h) * dv, work);
  }
}

int oracle_prefill_varlen(int64_t num_seqs, const int32_t* cu, int64_t hk, int64_t hv,
                          int64_t dk, int64_t dv, const void* q, const void* k, const void* v,
                          int in_dt, int64_t q_rs, int64_t k_rs, int64_t v_rs,
                          const double* g, const float* beta, int64_t beta_rs,
                          const void* pool, int state_dt, int64_t num_slots,
                          const int32_t* idx,
                          const int8_t* has_init, double scale, double l2_eps, int l2norm,
                          const uint8_t* head_mask, double* out, double* state_out) {
  int rc = check_common(hk, hv, dk, dv, scale);
  if (rc) return rc;
  if (state_dt != OR_F32 && state_dt != OR_F16 && state_dt != OR_BF16) return OR_ERR_ARG;
  if (num_seqs < 0 || cu[0] != 0) return OR_ERR_SHAPE;
  for (int64_t s = 0; s < num_seqs; ++s)
    if (cu[s + 1] < cu[s]) return OR_ERR_SHAPE;
  if (idx) {
    rc = check_slots(idx, num_seqs, num_slots, 0);
    if (rc) return rc;
  } else if (num_seqs > num_slots) {
    return OR_ERR_SLOT;
  }
  const struct prefill_ctx c = {cu, hk, hv, dk, dv, hv / hk, q, k, v, in_dt, q_rs, k_rs, v_rs,
                                g, beta, beta_rs, pool, state_dt, idx, has_init, scale, l2_eps,
                                l2norm, head_mask, out, state_out};
  return run_units(prefill_unit, &c, num_seqs * hv, (size_t)(2 * dk + 2 * dv));
}

/* ------------------------------------------------------------------------
 * Gated RMSNorm (vllm.cpp "rmsnorm_gated: norm-then-gate, silu and sigmoid
 * activations"; the rank-3 padded-row gate case).  For each token t and
 * v-head h, with x the [dv] row x[t][h]:
 *   ms      = (1/dv) sum_i x_i^2             (a mean, not a sum)
 *   y_i     = x_i / sqrt(ms + eps) * w_i * act(z[t][h][i])
 *   act     = silu(z) = z / (1 + exp(-z))   (default)
 *             sigmoid(z) = 1 / (1 + exp(-z)) (sigmoid != 0)
 * Normalise first, then gate.  x: [rows][hv][dv] (x_dt, OR_F64 allowed);
 * z: row t's gate at z[t * z_row_stride + h * dv + i] (a padded token row);
 * w: [dv].  y: [rows][hv][dv] f64.
 * ------------------------------------------------------------------------ */
static double act_gate(double z, int sigmoid) {
  const double sg = 1.0 / (1.0 + exp(-z));
  return sigmoid ? sg : z * sg;
}

int oracle_rmsnorm_gated(int64_t rows, int64_t hv, int64_t dv, const void* x, int x_dt,
                         const void* z, int z_dt, int64_t z_row_stride, const void* w,
                         int w_dt, double eps, int sigmoid, double* y) {
  if (rows < 0 || hv <= 0 || dv <= 0 || z_row_stride < hv * dv) return OR_ERR_SHAPE;
  if (!(eps >= 0.0)) return OR_ERR_ARG;
  for (int64_t t = 0; t < rows; ++t) {
    for (int64_t h = 0; h < hv; ++h) {
      const int64_t xo = (t * hv + h) * dv;
      double ms = 0.0;
      for (int64_t i = 0; i < dv; ++i) {
        const double xi = load_elem(x, x_dt, xo + i);
        ms += xi * xi;
      }
      ms /= (double)dv;
      const double inv = 1.0 / sqrt(ms + eps);
      for (int64_t i = 0; i < dv; ++i) {
        const double xi = load_elem(x, x_dt, xo + i);
        const double zi = load_elem(z, z_dt, t * z_row_stride + h * dv + i);
        y[xo + i] = xi * inv * load_elem(w, w_dt, i) * act_gate(zi, sigmoid);
      }
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------------
 * Rounding a binary32 value through a 16-bit storage format (nearest, ties to
 * even), returned widened.  Written from the format definitions:
 *  bfloat16 keeps the top 16 bits of the binary32 pattern;
 *  binary16 has a quantum of 2^(e-10) for 2^-14 <= |x| (e = floor(log2|x|)),
 *  2^-24 below that, and overflows to infinity past 65504.
 * ------------------------------------------------------------------------ */
static double round_through(float x, int dt) {
  if (dt == OR_F32 || isnan(x) || isinf(x)) return (double)x;
  if (dt == OR_BF16) {
    uint32_t u;
    memcpy(&u, &x, 4);
    const uint32_t lsb = (u >> 16) & 1u;
    u = (u + 0x7fffu + lsb) & 0xffff0000u;
    float r;
    memcpy(&r, &u, 4);
    return (double)r;
  }
  /* binary16 */
  const double ax = fabs((double)x);
  if (ax == 0.0) return (double)x;
  const int e = ilogb(ax);
  const double quantum = e < -14 ? ldexp(1.0, -24) : ldexp(1.0, e - 10);
  double r = nearbyint(ax / quantum) * quantum; /* default mode: ties to even */
  if (r > 65504.0) r = INFINITY;
  return x < 0 ? -r : r;
}

/* The pages' beta: the logistic function evaluated in binary32. */
static float sigmoid_f32(float b) { return 1.0f / (1.0f + expf(-b)); }

/* exported so the tests can pin the rounding against the format definitions */
double oracle_round_through(float x, int dt) { return round_through(x, dt); }

/* ------------------------------------------------------------------------
 * Gate and beta from raw projections (vllm.cpp "GdnGBeta"; the packed
 * in_proj_ba case: a and b are column views of one merged row, each with its
 * own row stride and offset, in one dtype):
 *   g    = softplus(a + dt_bias) * ssm_a             (as oracle_gate)
 *   beta = sigmoid(b)                                 (round_beta == 0)
 *        = sigmoid(b) rounded through b's dtype       (round_beta != 0,
 *          PackedDecodeReference)
 * sigmoid in binary32 as the pages compute it; g and beta returned in f64.
 * ------------------------------------------------------------------------ */
int oracle_gate_beta(int64_t rows, int64_t hv, const void* a, const void* b, int ab_dt,
                     int64_t a_row_stride, int64_t b_row_stride, const float* dt_bias,
                     const float* ssm_a, int round_beta, double* g, double* beta) {
  if (rows < 0 || hv <= 0 || a_row_stride < hv || b_row_stride < hv) return OR_ERR_SHAPE;
  if (ab_dt != OR_F32 && ab_dt != OR_F16 && ab_dt != OR_BF16) return OR_ERR_ARG;
  int rc = oracle_gate(rows, hv, a, ab_dt, a_row_stride, dt_bias, ssm_a, g);
  if (rc) return rc;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t h = 0; h < hv; ++h) {
      const float bv = (float)load_elem(b, ab_dt, r * b_row_stride + h);
      const float s = sigmoid_f32(bv);
      beta[r * hv + h] = round_beta ? round_through(s, ab_dt) : (double)s;
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------------
 * Post-conv front-end (vllm.cpp "gdn_post_conv fused == composed"): token t's
 * conv output row (conv_dt, row stride conv_row_stride) holds q in columns
 * [0, Hk*Dk), k in [Hk*Dk, 2*Hk*Dk) and v in [2*Hk*Dk, 2*Hk*Dk + Hv*Dv).
 *   q_out, k_out [T][Hk][Dk]: x / sqrt(sum x^2 + l2_eps) per head (no scale)
 *   v_out [T][Hv][Dv]: copied
 *   g, beta [T][Hv]: oracle_gate_beta with round_beta = 0
 * All outputs f64.
 * ------------------------------------------------------------------------ */
int oracle_post_conv(int64_t T, int64_t hk, int64_t hv, int64_t dk, int64_t dv,
                     const void* conv, int conv_dt, int64_t conv_row_stride, const void* a,
                     const void* b, int ab_dt, int64_t a_row_stride, int64_t b_row_stride,
                     const float* dt_bias, const float* ssm_a, double l2_eps, double* q_out,
                     double* k_out, double* v_out, double* g, double* beta) {
  if (T < 0 || hk <= 0 || hv <= 0 || dk <= 0 || dv <= 0) return OR_ERR_SHAPE;
  if (conv_row_stride < 2 * hk * dk + hv * dv) return OR_ERR_SHAPE;
  for (int64_t t = 0; t < T; ++t) {
    const int64_t row = t * conv_row_stride;
    for (int64_t h = 0; h < hk; ++h) {
      double* qo = q_out + (t * hk + h) * dk;
      double* ko = k_out + (t * hk + h) * dk;
      for (int64_t j = 0; j < dk; ++j) {
        qo[j] = load_elem(conv, conv_dt, row + h * dk + j);
        ko[j] = load_elem(conv, conv_dt, row + hk * dk + h * dk + j);
      }
      l2_normalize(qo, dk, l2_eps);
      l2_normalize(ko, dk, l2_eps);
    }
    for (int64_t i = 0; i < hv * dv; ++i)
      v_out[t * hv * dv + i] = load_elem(conv, conv_dt, row + 2 * hk * dk + i);
  }
  return oracle_gate_beta(T, hv, a, b, ab_dt, a_row_stride, b_row_stride, dt_bias, ssm_a, 0, g,
                          beta);
}

/* ------------------------------------------------------------------------
 * Depthwise causal conv1d (vllm.cpp "causal_conv1d_fwd: bias + initial state,
 * hand-computed", the short-sequence write-back case, "causal_conv1d_update:
 * bias + rolling state", the indexed, widened-cache and padded-row cases).
 * For channel c with taps w[c][0..K-1] (w[c][K-1] multiplies the current
 * token) and the token's window (the K-1 inputs before it, then itself):
 *   y = act(bias[c] + sum_j w[c][j] * window[j]),   act = silu or identity
 * The state holds the K-1 raw (pre-activation) inputs before the next token;
 * slot s's row for channel c starts at state[(s * C + c) * state_len]
 * (state_len >= K-1; only the leading K-1 entries are used).
 * Storage: x, w, bias in x_dt; state in st_dt (read widened, returned f64).
 * ------------------------------------------------------------------------ */
static double conv_act(double v, int silu) { return silu ? v / (1.0 + exp(-v)) : v; }

/* Varlen forward.  Sequence s covers tokens [cu[s], cu[s+1]); its window
 * before its first token is state row idx[s] (idx NULL: s) when has_init[s]
 * (NULL: all 1), else zeros.  out [T][C] f64; state_out [num_seqs][C][K-1]
 * f64: the last K-1 entries of (initial window, then the sequence's inputs). */
int oracle_conv1d_fwd(int64_t num_seqs, const int32_t* cu, int64_t C, int64_t K,
                      const void* x, int x_dt, int64_t x_row_stride, const void* w,
                      const void* bias, const void* state, int st_dt, int64_t state_len,
                      int64_t num_slots, const int32_t* idx, const int8_t* has_init, int silu,
                      double* out, double* state_out) {
  if (num_seqs < 0 || C <= 0 || K <= 0 || x_row_stride < C || state_len < K - 1)
    return OR_ERR_SHAPE;
  if (cu[0] != 0) return OR_ERR_SHAPE;
  for (int64_t s = 0; s < num_seqs; ++s)
    if (cu[s + 1] < cu[s]) return OR_ERR_SHAPE;
  if (idx) {
    int rc = check_slots(idx, num_seqs, num_slots, 0);
    if (rc) return rc;
  } else if (num_seqs > num_slots) {
    return OR_ERR_SLOT;
  }
  double* win = (double*)malloc((size_t)K * sizeof(double));
  if (!win) return OR_ERR_ARG;
  for (int64_t s = 0; s < num_seqs; ++s) {
    const int64_t slot = idx ? idx[s] : s;
    const int init = has_init ? has_init[s] != 0 : 1;
    for (int64_t c = 0; c < C; ++c) {
      /* win[0..K-2]: the K-1 inputs before the current token */
      for (int64_t j = 0; j < K - 1; ++j)
        win[j] = init ? load_elem(state, st_dt, (slot * C + c) * state_len + j) : 0.0;
      const double wc_last = load_elem(w, x_dt, c * K + K - 1);
      const double b = bias ? load_elem(bias, x_dt, c) : 0.0;
      for (int64_t t = cu[s]; t < cu[s + 1]; ++t) {
        const double xt = load_elem(x, x_dt, t * x_row_stride + c);
        double acc = b;
        for (int64_t j = 0; j < K - 1; ++j) acc += load_elem(w, x_dt, c * K + j) * win[j];
        acc += wc_last * xt;
        out[t * C + c] = conv_act(acc, silu);
        for (int64_t j = 0; j + 1 < K - 1; ++j) win[j] = win[j + 1];
        if (K > 1) win[K - 2] = xt;
      }
      for (int64_t j = 0; j < K - 1; ++j) state_out[(s * C + c) * (K - 1) + j] = win[j];
    }
  }
  free(win);
  return OR_OK;
}

/* Single-token update for `batch` rows: row r uses state slot idx[r] (idx
 * NULL: r); a negative slot leaves its output row and every state alone (the
 * caller's out is then kept, and out_written[r] = 0).  out [batch][C] f64;
 * state_out [batch][C][K-1] f64: the rolled window (old entries shifted left,
 * the raw input appended). */
int oracle_conv1d_update(int64_t batch, int64_t C, int64_t K, const void* x, int x_dt,
                         int64_t x_row_stride, const void* w, const void* bias,
                         const void* state, int st_dt, int64_t state_len, int64_t num_slots,
                         const int32_t* idx, int silu, double* out, double* state_out,
                         int8_t* out_written) {
  if (batch < 0 || C <= 0 || K <= 0 || x_row_stride < C || state_len < K - 1)
    return OR_ERR_SHAPE;
  if (idx) {
    int rc = check_slots(idx, batch, num_slots, 1);
    if (rc) return rc;
  } else if (batch > num_slots) {
    return OR_ERR_SLOT;
  }
  for (int64_t r = 0; r < batch; ++r) {
    const int64_t slot = idx ? idx[r] : r;
    out_written[r] = slot >= 0;
    if (slot < 0) continue;
    for (int64_t c = 0; c < C; ++c) {
      const int64_t srow = (slot * C + c) * state_len;
      const double xt = load_elem(x, x_dt, r * x_row_stride + c);
      double acc = bias ? load_elem(bias, x_dt, c) : 0.0;
      for (int64_t j = 0; j < K - 1; ++j)
        acc += load_elem(w, x_dt, c * K + j) * load_elem(state, st_dt, srow + j);
      acc += load_elem(w, x_dt, c * K + K - 1) * xt;
      out[r * C + c] = conv_act(acc, silu);
      double* so = state_out + (r * C + c) * (K - 1);
      for (int64_t j = 0; j + 1 < K - 1; ++j) so[j] = load_elem(state, st_dt, srow + j + 1);
      if (K > 1) so[K - 2] = xt;
    }
  }
  return OR_OK;
}
