// gdn_frontend.hip -- the post-conv front-end (vllm.cpp tests/vt/test_ops_gdn.cpp,
// "gdn_post_conv fused == composed"): each token row of the conv output holds
// q | k | v (q in columns [0, hk*dk), k in [hk*dk, 2*hk*dk), v after them);
// q and k are L2-normalised per head (no scale), v is copied, both converted
// to the output dtype.  g and beta come from gate_kernel (raw a/b views).
//
// Elementwise and HBM-bound: one 256-thread workgroup per token row.  The
// general form has each wave normalise whole q/k heads in turn (a 64-lane sum
// per head, one element per lane), then all threads copy the v segment.  The decode and prefill kernels read the
// conv output rows directly (row-strided q/k/v views, norm in-kernel), so
// this pass exists for callers that want q/k/v materialised.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

__global__ __launch_bounds__(256) void post_conv_kernel(PostConvArgs a) {
  const int64_t t = blockIdx.x;
  const int wid = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t row = t * a.conv_rs;
  // heads 0..hk-1 are q, hk..2hk-1 are k: contiguous dk-wide column blocks
  for (int j = wid; j < 2 * a.hk; j += 4) {
    const int64_t src = row + (int64_t)j * a.dk;
    float ss = 0.0f;
    for (int e = lane; e < a.dk; e += 64) {
      const float x = load1(a.conv, a.conv_dt, src + e);
      ss += x * x;
    }
    ss = group_sum<64>(ss);
    const float inv = 1.0f / sqrtf(ss + a.l2_eps);
    void* dst = j < a.hk ? a.q : a.k;
    const int64_t o = (t * a.hk + (j < a.hk ? j : j - a.hk)) * a.dk;
    for (int e = lane; e < a.dk; e += 64)
      store1(dst, a.out_dt, o + e, load1(a.conv, a.conv_dt, src + e) * inv);
  }
  const int64_t vw = (int64_t)a.hv * a.dv;
  const int64_t vsrc = row + 2 * (int64_t)a.hk * a.dk;
  for (int64_t e = threadIdx.x; e < vw; e += 256)
    store1(a.v, a.out_dt, t * vw + e, load1(a.conv, a.conv_dt, vsrc + e));
}

// Vector form, where the layout allows it: every lane moves 16 bytes of the
// input row (8 elements in 16-bit, 4 in f32).  The q | k columns are walked as
// one flat run of such pieces; a head's dk/VEC pieces sit on an aligned group
// of consecutive lanes (dk/VEC a power of two <= 64), whose sum of squares is
// one butterfly within the group.  The loop step is the workgroup width, a
// multiple of the group, so a group is always wholly inside or outside the run.
template <int TIN>
struct InVec;
template <>
struct InVec<kF32> {
  static constexpr int N = 4;
  __device__ static void load(const void* p, int64_t off, float* x) {
    const f32x4_t r = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p) + off));
    x[0] = r[0]; x[1] = r[1]; x[2] = r[2]; x[3] = r[3];
  }
};
template <int TIN>
struct InVec16 {
  static constexpr int N = 8;
  __device__ static void load(const void* p, int64_t off, float* x) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t r = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p) + off));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = TIN == kBF16 ? bf16_to_f32(r[i] & 0xffffu) : f16_to_f32(r[i] & 0xffffu);
      x[2 * i + 1] = TIN == kBF16 ? bf16_to_f32(r[i] >> 16) : f16_to_f32(r[i] >> 16);
    }
  }
};
template <>
struct InVec<kF16> : InVec16<kF16> {};
template <>
struct InVec<kBF16> : InVec16<kBF16> {};

// N elements (4 or 8) stored from f32 at element `off` of a TOUT array.
template <int TOUT, int N>
__device__ __forceinline__ void store_vec(void* p, int64_t off, const float* x) {
  if constexpr (TOUT == kF32) {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      *reinterpret_cast<float4*>(static_cast<float*>(p) + off + i) =
          make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
  } else {
    uint32_t w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i)
      w[i] = TOUT == kBF16 ? pack2_bf16(x[2 * i], x[2 * i + 1]) : pack2_f16(x[2 * i], x[2 * i + 1]);
    uint16_t* d = static_cast<uint16_t*>(p) + off;
    if constexpr (N == 8) *reinterpret_cast<uint4*>(d) = make_uint4(w[0], w[1], w[2], w[3]);
    else *reinterpret_cast<uint2*>(d) = make_uint2(w[0], w[1]);
  }
}

__device__ __forceinline__ float lane_group_sum(float v, int g) {
  switch (g) {
    case 1: return v;
    case 2: return group_sum<2>(v);
    case 4: return group_sum<4>(v);
    case 8: return group_sum<8>(v);
    case 16: return group_sum<16>(v);
    case 32: return group_sum<32>(v);
    default: return group_sum<64>(v);
  }
}

template <int TIN, int TOUT>
__global__ __launch_bounds__(256) void post_conv_vec_kernel(PostConvArgs a) {
  constexpr int N = InVec<TIN>::N;
  const int64_t t = blockIdx.x;
  const int64_t row = t * a.conv_rs;
  const int per_head = a.dk / N;        // lanes per head: a power of two <= 64
  const int nqk = 2 * a.hk * per_head;  // q then k pieces of this row
  for (int c = threadIdx.x; c < nqk; c += 256) {
    float x[N];
    InVec<TIN>::load(a.conv, row + (int64_t)c * N, x);
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i) ss += x[i] * x[i];
    ss = lane_group_sum(ss, per_head);
    const float inv = 1.0f / sqrtf(ss + a.l2_eps);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] *= inv;
    const int j = c / per_head;  // head among the 2*hk q and k heads
    const int e = (c - j * per_head) * N;
    void* dst = j < a.hk ? a.q : a.k;
    store_vec<TOUT, N>(dst, (t * a.hk + (j < a.hk ? j : j - a.hk)) * a.dk + e, x);
  }
  const int64_t vw = (int64_t)a.hv * a.dv;
  const int64_t vsrc = row + 2 * (int64_t)a.hk * a.dk;
  for (int64_t c = threadIdx.x; c * N < vw; c += 256) {
    float x[N];
    InVec<TIN>::load(a.conv, vsrc + c * N, x);
    store_vec<TOUT, N>(a.v, t * vw + c * N, x);
  }
}

template <int TIN>
void launch_vec(const PostConvArgs& a, hipStream_t stream) {
  const dim3 g((unsigned)a.T), b(256);
  if (a.out_dt == kF32) hipLaunchKernelGGL((post_conv_vec_kernel<TIN, kF32>), g, b, 0, stream, a);
  else if (a.out_dt == kF16) hipLaunchKernelGGL((post_conv_vec_kernel<TIN, kF16>), g, b, 0, stream, a);
  else hipLaunchKernelGGL((post_conv_vec_kernel<TIN, kBF16>), g, b, 0, stream, a);
}

bool post_conv_vec_ok(const PostConvArgs& a) {
  const int n = a.conv_dt == kF32 ? 4 : 8;
  const int ec = a.conv_dt == kF32 ? 4 : 2, eo = a.out_dt == kF32 ? 4 : 2;
  const int oa = n * eo < 16 ? n * eo : 16;
  const int per_head = a.dk / n;
  auto al = [](const void* p, int m) { return reinterpret_cast<uintptr_t>(p) % m == 0; };
  return a.dk % n == 0 && per_head <= 64 && (per_head & (per_head - 1)) == 0 &&
         ((int64_t)a.hv * a.dv) % n == 0 && (a.conv_rs * ec) % 16 == 0 && al(a.conv, 16) &&
         al(a.q, oa) && al(a.k, oa) && al(a.v, oa);
}

}  // namespace

hipError_t launch_post_conv(const PostConvArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  if (a.T >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (post_conv_vec_ok(a)) {
    if (a.conv_dt == kF32) launch_vec<kF32>(a, stream);
    else if (a.conv_dt == kF16) launch_vec<kF16>(a, stream);
    else launch_vec<kBF16>(a, stream);
  } else {
    hipLaunchKernelGGL(post_conv_kernel, dim3((unsigned)a.T), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace gdn
