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

// f32 -> bfloat16 / binary16, round to nearest even, converted in hardware
// (v_cvt_pk_bf16_f32, v_cvt_f16_f32).  On gfx950 the bf16 conversion gives
// exactly the rule above, NaN quieting included: checked on the device for
// the bit patterns of Winery-Strata's bf16_bits_test list (NaNs of both
// signs and payloads, infinities, the largest finite, ties, subnormals).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ uint16_t f32_to_f16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two values rounded and packed into one word, a in the low half.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

__device__ __forceinline__ uint32_t pack2_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, f16x2_t));
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

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 16-byte state access, optionally with the nontemporal (streaming) hint.
template <bool NT>
__device__ __forceinline__ float4 state_load(const float* p) {
  if constexpr (NT) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
  } else {
    return *reinterpret_cast<const float4*>(p);
  }
}

template <bool NT>
__device__ __forceinline__ void state_store(float* p, float4 x) {
  if constexpr (NT) {
    f32x4_t v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
  } else {
    *reinterpret_cast<float4*>(p) = x;
  }
}

// Four consecutive state elements in storage dtype TS (f32, binary16 or
// bfloat16), widened to f32 on load and rounded to nearest-even on store.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int TS, bool NT>
__device__ __forceinline__ float4 state_load4(const void* base, int64_t off) {
  if constexpr (TS == kF32) {
    return state_load<NT>(static_cast<const float*>(base) + off);
  } else {
    const u32x2_t* p = reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(base) + off);
    u32x2_t r;
    if constexpr (NT) r = __builtin_nontemporal_load(p);
    else r = *p;
    const uint32_t lo = r[0], hi = r[1];
    if constexpr (TS == kBF16)
      return make_float4(bf16_to_f32(lo & 0xffffu), bf16_to_f32(lo >> 16),
                         bf16_to_f32(hi & 0xffffu), bf16_to_f32(hi >> 16));
    else
      return make_float4(f16_to_f32(lo & 0xffffu), f16_to_f32(lo >> 16),
                         f16_to_f32(hi & 0xffffu), f16_to_f32(hi >> 16));
  }
}

template <int TS, bool NT>
__device__ __forceinline__ void state_store4(void* base, int64_t off, float4 x) {
  if constexpr (TS == kF32) {
    state_store<NT>(static_cast<float*>(base) + off, x);
  } else {
    u32x2_t r;
    if constexpr (TS == kBF16) r = u32x2_t{pack2_bf16(x.x, x.y), pack2_bf16(x.z, x.w)};
    else r = u32x2_t{pack2_f16(x.x, x.y), pack2_f16(x.z, x.w)};
    u32x2_t* p = reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(base) + off);
    if constexpr (NT) __builtin_nontemporal_store(r, p);
    else *p = r;
  }
}

// The same with the storage dtype known only at run time (state loaded or
// stored once per kernel, outside any loop).
__device__ __forceinline__ float4 state_load4_rt(int ts, const void* base, int64_t off) {
  if (ts == kBF16) return state_load4<kBF16, false>(base, off);
  if (ts == kF16) return state_load4<kF16, false>(base, off);
  return state_load4<kF32, false>(base, off);
}

__device__ __forceinline__ void state_store4_rt(int ts, void* base, int64_t off, float4 x) {
  if (ts == kBF16) state_store4<kBF16, false>(base, off, x);
  else if (ts == kF16) state_store4<kF16, false>(base, off, x);
  else state_store4<kF32, false>(base, off, x);
}

// Gate activation of the gated RMSNorm: silu(z) = z * sigmoid(z), or sigmoid(z),
// with sigmoid(z) = 1 / (1 + 2^(-z log2 e)) on the hardware base-2 exponential
// and reciprocal (about 1 ulp each).  One implementation for the norm fused
// into decode and the standalone norm, so the same o and z give the same
// result on both paths.  The library expf and an IEEE division made the
// standalone pass ALU-bound (149 -> 99 us over the [32768, 24, 128] fp16
// prefill output).
__device__ __forceinline__ float gate_act(float z, bool sigmoid) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
  return sigmoid ? sg : z * sg;
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

// Butterfly partner exchange for bit M (a power of two <= 32): returns the
// value of a lane whose bit M is flipped and whose bits above M are equal.
// Bits below M may be flipped too (the mirrors below map lane l to l ^ (2M-1)),
// which is all a butterfly reduction needs: at each step the partner sits on
// the other side of bit M and holds partial sums over the same rows, and the
// partners met over all steps still cover each lane exactly once.
//   M = 1, 2: DPP quad_perm;  M = 4: DPP row_half_mirror (l ^ 7);
//   M = 8: DPP row_mirror (l ^ 15);  M = 16: ds_swizzle xor within 32 lanes;
//   M = 32: ds_bpermute.
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  const int x = __float_as_int(v);
  if constexpr (M == 1) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
  } else if constexpr (M == 2) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
  } else if constexpr (M == 4) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false));
  } else if constexpr (M == 8) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false));
  } else if constexpr (M == 16) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x401F));
  } else {
    static_assert(M == 32, "xor_lane: M must be a power of two <= 32");
    return __shfl_xor(v, 32, 64);
  }
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

// Typed raw loads.  The raw bits are loaded first and converted later, so a
// kernel can issue all of its loads back to back before waiting on any of
// them (a conversion right after a load would force an early wait).
template <int DT>
struct Raw4 {
  uint32_t w[DT == kF32 ? 4 : 2];
};

template <int DT>
__device__ __forceinline__ Raw4<DT> load_raw4(const void* p, int64_t off, bool vec) {
  Raw4<DT> r;
  if constexpr (DT == kF32) {
    const uint32_t* q = static_cast<const uint32_t*>(p) + off;
    if (vec) {
      const uint4 u = *reinterpret_cast<const uint4*>(q);
      r.w[0] = u.x; r.w[1] = u.y; r.w[2] = u.z; r.w[3] = u.w;
    } else {
      r.w[0] = q[0]; r.w[1] = q[1]; r.w[2] = q[2]; r.w[3] = q[3];
    }
  } else {
    const uint16_t* q = static_cast<const uint16_t*>(p) + off;
    if (vec) {
      const uint2 u = *reinterpret_cast<const uint2*>(q);
      r.w[0] = u.x; r.w[1] = u.y;
    } else {
      r.w[0] = (uint32_t)q[0] | ((uint32_t)q[1] << 16);
      r.w[1] = (uint32_t)q[2] | ((uint32_t)q[3] << 16);
    }
  }
  return r;
}

template <int DT>
__device__ __forceinline__ float4 raw_to_f32(const Raw4<DT>& r) {
  if constexpr (DT == kF32) {
    return make_float4(__uint_as_float(r.w[0]), __uint_as_float(r.w[1]),
                       __uint_as_float(r.w[2]), __uint_as_float(r.w[3]));
  } else if constexpr (DT == kBF16) {
    return make_float4(bf16_to_f32(r.w[0] & 0xffffu), bf16_to_f32(r.w[0] >> 16),
                       bf16_to_f32(r.w[1] & 0xffffu), bf16_to_f32(r.w[1] >> 16));
  } else {
    return make_float4(f16_to_f32(r.w[0] & 0xffffu), f16_to_f32(r.w[0] >> 16),
                       f16_to_f32(r.w[1] & 0xffffu), f16_to_f32(r.w[1] >> 16));
  }
}

template <int DT>
__device__ __forceinline__ uint32_t load_raw1(const void* p, int64_t off) {
  if constexpr (DT == kF32) return static_cast<const uint32_t*>(p)[off];
  return static_cast<const uint16_t*>(p)[off];
}

template <int DT>
__device__ __forceinline__ float raw1_to_f32(uint32_t u) {
  if constexpr (DT == kF32) return __uint_as_float(u);
  if constexpr (DT == kBF16) return bf16_to_f32(u);
  return f16_to_f32(u);
}

// softplus with the large-x branch, then times ssm_a (negative): the gate g.
__device__ __forceinline__ float gate_value(float x, float ssm_a) {
  const float sp = x > 20.0f ? x : log1pf(expf(x));
  return sp * ssm_a;
}

// beta from the raw projection b: the logistic function in f32, optionally
// rounded through b's 16-bit storage format (nearest even) and widened back.
template <int DT>
__device__ __forceinline__ float beta_from_raw(float b, bool round) {
  const float s = 1.0f / (1.0f + expf(-b));
  if constexpr (DT == kBF16) return round ? bf16_to_f32(f32_to_bf16(s)) : s;
  else if constexpr (DT == kF16) return round ? f16_to_f32(f32_to_f16(s)) : s;
  else return s;
}

// beta from the raw b, the storage format chosen at run time
__device__ __forceinline__ float beta_from_raw_rt(float b, int dt, bool round) {
  return dt == kBF16 ? beta_from_raw<kBF16>(b, round)
         : dt == kF16 ? beta_from_raw<kF16>(b, round)
                      : beta_from_raw<kF32>(b, round);
}

}  // namespace gdn
