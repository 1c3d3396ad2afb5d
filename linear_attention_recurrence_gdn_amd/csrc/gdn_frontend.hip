// gdn_frontend.hip -- the post-conv front-end (vllm.cpp tests/vt/test_ops_gdn.cpp,
// "gdn_post_conv fused == composed"): each token row of the conv output holds
// q | k | v (q in columns [0, hk*dk), k in [hk*dk, 2*hk*dk), v after them);
// q and k are L2-normalised per head (no scale), v is copied, both converted
// to the output dtype.  g and beta come from gate_kernel (raw a/b views).
//
// Elementwise and HBM-bound: one 256-thread workgroup per token row, each
// wave normalising whole q/k heads in turn (a 64-lane sum per head), then all
// threads copying the v segment.  The decode and prefill kernels read the
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

}  // namespace

hipError_t launch_post_conv(const PostConvArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  if (a.T >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(post_conv_kernel, dim3((unsigned)a.T), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
