// gdn_prefill_gate.h -- the gate and beta of one (token, v-head) for the
// prefill kernels: read from the materialised g and beta, or formed in the
// kernel from the raw gate inputs with the arithmetic of gate_kernel
// (g = softplus(alpha + dt_bias) * ssm_a with the x > 20 branch; beta =
// sigmoid(b), optionally rounded through b's dtype), so both routes give the
// same bits (Winery-Strata elementwise_parity.cpp, the gdn_gate block;
// vllm.cpp test_ops_gdn.cpp, GdnGBeta and PackedDecodeReference's beta).
#pragma once

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

__device__ __forceinline__ void token_gate(const PrefillArgs& a, int64_t t, int h, float& g,
                                           float& beta) {
  if (a.alpha)
    g = gate_value(load1(a.alpha, a.alpha_dt, t * a.alpha_rs + h) + a.dt_bias[h], a.ssm_a[h]);
  else
    g = a.g[t * a.g_rs + h];
  if (a.beta_raw)
    beta = beta_from_raw_rt(load1(a.beta, a.alpha_dt, t * a.beta_rs + h), a.alpha_dt,
                            a.round_beta != 0);
  else
    beta = static_cast<const float*>(a.beta)[t * a.beta_rs + h];
}

}  // namespace gdn
