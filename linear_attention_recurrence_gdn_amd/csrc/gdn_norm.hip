// gdn_norm.hip -- gated RMSNorm over the recurrence output (vllm.cpp
// tests/vt/test_ops_gdn.cpp, "rmsnorm_gated: norm-then-gate, silu and sigmoid
// activations" and the rank-3 padded-row gate case):
//   out[t][h][i] = x[t][h][i] / sqrt(mean_i x^2 + eps) * w[i] * act(z[t][h][i])
// with act = silu (default) or sigmoid, normalise first, then gate.
//
// HBM-bound elementwise work with one reduction per (token, v-head) row:
// each lane owns N consecutive elements of a row, 16 bytes of x and of z
// (N = 8 for 16-bit data, 4 for f32), G = dv / N lanes share a row, and a
// wave takes RPL = 4 row groups per pass with every load issued before any
// arithmetic (128 bytes per lane in flight).  Rows whose dv / N is not a
// power of two <= 64 go through a plain wave-per-row loop.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kRpl = 4;   // row groups per wave pass

template <int DT>
struct V16 {
  static constexpr int N = DT == kF32 ? 4 : 8;   // elements in 16 bytes
  static constexpr int EB = DT == kF32 ? 4 : 2;
};

// x and z are read once and the output written once: every access carries
// the nontemporal (streaming) hint, except the weight row, which all rows share.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ uint4 ld16(const void* p, int64_t elem) {
  return *reinterpret_cast<const uint4*>(static_cast<const char*>(p) + elem * V16<DT>::EB);
}

template <int DT>
__device__ __forceinline__ uint4 ld16_stream(const void* p, int64_t elem) {
  const u32x4_t r = __builtin_nontemporal_load(
      reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p) + elem * V16<DT>::EB));
  return make_uint4(r[0], r[1], r[2], r[3]);
}

template <int DT>
__device__ __forceinline__ void widen16(uint4 u, float (&v)[V16<DT>::N]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  if constexpr (DT == kF32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = DT == kBF16 ? bf16_to_f32(w[i] & 0xffffu) : f16_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = DT == kBF16 ? bf16_to_f32(w[i] >> 16) : f16_to_f32(w[i] >> 16);
    }
  }
}

// N outputs of one lane: f32 (OF32) or rounded to the 16-bit input format.
template <int DT, bool OF32>
__device__ __forceinline__ void st_out(void* p, int64_t elem, const float (&y)[V16<DT>::N]) {
  constexpr int N = V16<DT>::N;
  if constexpr (OF32 || DT == kF32) {
    float* o = static_cast<float*>(p) + elem;
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const f32x4_t r = {y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]};
      __builtin_nontemporal_store(r, reinterpret_cast<f32x4_t*>(o + 4 * i));
    }
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = DT == kBF16 ? pack2_bf16(y[2 * i], y[2 * i + 1]) : pack2_f16(y[2 * i], y[2 * i + 1]);
    const u32x4_t r = {w[0], w[1], w[2], w[3]};
    __builtin_nontemporal_store(r, reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p) + elem));
  }
}

template <int G, int DT, bool OF32>
__global__ __launch_bounds__(256) void rmsnorm_gated_kernel(NormArgs a, int64_t nrows) {
  constexpr int N = V16<DT>::N;
  constexpr int DV = G * N;
  constexpr int RPW = 64 / G;               // rows per wave per group
  const int lane = threadIdx.x & 63;
  const int col = (lane % G) * N;
  const int sub = lane / G;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t r0 = wave * (RPW * kRpl);
  if (r0 >= nrows) return;

  uint4 xr[kRpl], zr[kRpl];
#pragma unroll
  for (int u = 0; u < kRpl; ++u) {
    const int64_t r = min(r0 + u * RPW + sub, nrows - 1);   // r = t * hv + h
    const int64_t t = r / a.hv;
    const int64_t h = r - t * a.hv;
    xr[u] = ld16_stream<DT>(a.x, r * DV + col);
    zr[u] = ld16_stream<DT>(a.z, t * a.z_rs + h * DV + col);
  }
  float w[N];
  widen16<DT>(ld16<DT>(a.w, col), w);
  const bool sig = a.sigmoid != 0;
#pragma unroll
  for (int u = 0; u < kRpl; ++u) {
    const int64_t r = r0 + u * RPW + sub;
    float x[N], z[N];
    widen16<DT>(xr[u], x);
    widen16<DT>(zr[u], z);
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i) ss += x[i] * x[i];
    ss = group_sum<G>(ss);
    const float inv = 1.0f / sqrtf(ss / (float)DV + a.eps);
    float y[N];
#pragma unroll
    for (int i = 0; i < N; ++i) y[i] = x[i] * inv * w[i] * gate_act(z[i], sig);
    if (r < nrows) st_out<DT, OF32>(a.out, r * DV + col, y);
  }
}

// Any dv: one wave per row, lanes strided over the row.
__global__ __launch_bounds__(256) void rmsnorm_gated_rows_kernel(NormArgs a, int64_t nrows) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= nrows) return;
  const int64_t t = r / a.hv;
  const int64_t h = r - t * a.hv;
  float ss = 0.0f;
  for (int i = lane; i < a.dv; i += 64) {
    const float x = load1(a.x, a.x_dt, r * a.dv + i);
    ss += x * x;
  }
  ss = group_sum<64>(ss);
  const float inv = 1.0f / sqrtf(ss / (float)a.dv + a.eps);
  const bool sig = a.sigmoid != 0;
  for (int i = lane; i < a.dv; i += 64) {
    const float x = load1(a.x, a.x_dt, r * a.dv + i);
    const float z = load1(a.z, a.x_dt, t * a.z_rs + h * a.dv + i);
    store1(a.out, a.out_dt, r * a.dv + i, x * inv * load1(a.w, a.x_dt, i) * gate_act(z, sig));
  }
}

template <int DT, bool OF32>
hipError_t launch_dt(const NormArgs& a, int64_t nrows, int g, hipStream_t stream) {
  const int per_wave = (64 / g) * kRpl;
  const int64_t waves = (nrows + per_wave - 1) / per_wave;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  switch (g) {
#define GDN_NORM_G(G) \
    case G: \
      hipLaunchKernelGGL((rmsnorm_gated_kernel<G, DT, OF32>), dim3((unsigned)blocks), dim3(256), \
                         0, stream, a, nrows); \
      return hipGetLastError();
    GDN_NORM_G(1) GDN_NORM_G(2) GDN_NORM_G(4) GDN_NORM_G(8) GDN_NORM_G(16) GDN_NORM_G(32)
    GDN_NORM_G(64)
#undef GDN_NORM_G
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// The vector path: dv a multiple of N (16 bytes of elements) with dv / N a
// power of two <= 64, the gate row stride a multiple of N, and every
// pointer 16-byte aligned.
static int norm_vec_groups(const NormArgs& a) {
  const int n = a.x_dt == kF32 ? 4 : 8;
  const int g = a.dv / n;
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) % 16) == 0; };
  if (a.dv % n != 0 || g < 1 || g > 64 || (g & (g - 1)) != 0 || a.z_rs % n != 0) return 0;
  if (!al(a.x) || !al(a.z) || !al(a.w) || !al(a.out)) return 0;
  return g;
}

hipError_t launch_rmsnorm_gated(const NormArgs& a, hipStream_t stream) {
  const int64_t nrows = a.rows * a.hv;
  if (nrows == 0) return hipSuccess;
  const int g = norm_vec_groups(a);
  if (g > 0) {
    const bool of32 = a.out_dt == kF32;
    if (a.x_dt == kF32) return launch_dt<kF32, true>(a, nrows, g, stream);
    if (a.x_dt == kBF16)
      return of32 ? launch_dt<kBF16, true>(a, nrows, g, stream)
                  : launch_dt<kBF16, false>(a, nrows, g, stream);
    if (a.x_dt == kF16)
      return of32 ? launch_dt<kF16, true>(a, nrows, g, stream)
                  : launch_dt<kF16, false>(a, nrows, g, stream);
    return hipErrorInvalidValue;
  }
  const int64_t blocks = (nrows + 3) / 4;
  if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rmsnorm_gated_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a,
                     nrows);
  return hipGetLastError();
}

}  // namespace gdn
