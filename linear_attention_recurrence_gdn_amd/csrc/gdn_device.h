// gdn_device.h -- device-side helpers shared by the GDN kernels (gfx950, wave64).
//
// Storage formats: f32; IEEE binary16; bfloat16 (the top half of a binary32).
// Outputs are rounded to nearest-even on store; a NaN stays a NaN (for bf16
// its top bits are kept with the quiet bit set, the rule Winery-Strata's
// f32_to_bf16_bulk check states).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

enum : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  const uint32_t b = __float_as_uint(x);
  if ((b & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((b >> 16) | 0x40u);
  return static_cast<uint16_t>((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// Four consecutive elements starting at element `off` (16-byte aligned for f32,
// 8-byte aligned for the 16-bit formats).
__device__ __forceinline__ float4 load4(const void* p, int dt, int64_t off) {
  if (dt == kF32) return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + off);
  const uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + off);
  if (dt == kBF16)
    return make_float4(bf16_to_f32(raw.x & 0xffffu), bf16_to_f32(raw.x >> 16),
                       bf16_to_f32(raw.y & 0xffffu), bf16_to_f32(raw.y >> 16));
  return make_float4(f16_to_f32(raw.x & 0xffffu), f16_to_f32(raw.x >> 16),
                     f16_to_f32(raw.y & 0xffffu), f16_to_f32(raw.y >> 16));
}

__device__ __forceinline__ float load1(const void* p, int dt, int64_t off) {
  if (dt == kF32) return static_cast<const float*>(p)[off];
  const uint32_t u = static_cast<const uint16_t*>(p)[off];
  return dt == kBF16 ? bf16_to_f32(u) : f16_to_f32(u);
}

// Four consecutive elements with no alignment requirement when !vec.
__device__ __forceinline__ float4 load4u(const void* p, int dt, int64_t off, bool vec) {
  if (vec) return load4(p, dt, off);
  return make_float4(load1(p, dt, off), load1(p, dt, off + 1), load1(p, dt, off + 2),
                     load1(p, dt, off + 3));
}

__device__ __forceinline__ void store1(void* p, int dt, int64_t off, float x) {
  if (dt == kF32) {
    static_cast<float*>(p)[off] = x;
  } else {
    static_cast<uint16_t*>(p)[off] = dt == kBF16 ? f32_to_bf16(x) : f32_to_f16(x);
  }
}

__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

__device__ __forceinline__ float4 axpby4(float a, float4 x, float b, float4 y) {
  return make_float4(a * x.x + b * y.x, a * x.y + b * y.y, a * x.z + b * y.z, a * x.w + b * y.w);
}

__device__ __forceinline__ float4 scale4(float a, float4 x) {
  return make_float4(a * x.x, a * x.y, a * x.z, a * x.w);
}

// Cross-lane exchange with lane ^ M inside the wavefront.
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  return __shfl_xor(v, M, 64);
}

// Full sum over aligned groups of G lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += xor_lane<1>(v);
  if constexpr (G >= 4) v += xor_lane<2>(v);
  if constexpr (G >= 8) v += xor_lane<4>(v);
  if constexpr (G >= 16) v += xor_lane<8>(v);
  if constexpr (G >= 32) v += xor_lane<16>(v);
  if constexpr (G >= 64) v += xor_lane<32>(v);
  return v;
}

// Transposed reduction of N partial sums per lane over aligned groups of G
// lanes (N <= G, both powers of two).  Each halving step trades half of the
// values with the partner lane, so the whole reduction costs N-1+log2(G/N)
// exchanges instead of N*log2(G).  On return a[0] holds, in every lane, the
// group-wide sum of value index (lane % G) / (G / N).
template <int N, int OFF>
__device__ __forceinline__ void transpose_reduce_step(float* a, int lane) {
  if constexpr (OFF >= 1) {
    if constexpr (N > 1) {
      const bool upper = (lane & OFF) != 0;
#pragma unroll
      for (int j = 0; j < N / 2; ++j) {
        const float send = upper ? a[j] : a[j + N / 2];
        const float keep = upper ? a[j + N / 2] : a[j];
        a[j] = keep + xor_lane<OFF>(send);
      }
      transpose_reduce_step<N / 2, OFF / 2>(a, lane);
    } else {
      a[0] += xor_lane<OFF>(a[0]);
      transpose_reduce_step<1, OFF / 2>(a, lane);
    }
  }
}

template <int N, int G>
__device__ __forceinline__ void transpose_reduce(float* a, int lane) {
  static_assert(N <= G, "transpose_reduce needs N <= G");
  transpose_reduce_step<N, G / 2>(a, lane);
}

// softplus with the large-x branch, then times ssm_a (negative): the gate g.
__device__ __forceinline__ float gate_value(float x, float ssm_a) {
  const float sp = x > 20.0f ? x : log1pf(expf(x));
  return sp * ssm_a;
}

}  // namespace gdn
