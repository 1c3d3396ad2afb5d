// gdn_conv.hip -- depthwise causal conv1d before the GDN front-end (vllm.cpp
// tests/vt/test_ops_gdn.cpp, the causal_conv1d_fwd / causal_conv1d_update
// cases): for channel c with taps w[c][0..K-1], the last on the current token,
//   y = act(bias[c] + sum_j w[c][j] * window[j]),  act = silu or identity,
// where the window is the K-1 inputs before the token, then the token.  The
// state row of a sequence holds the K-1 raw inputs before its next token.
//
// Forward (varlen prefill): HBM-bound, read x once and write y once.  Each
// thread owns one channel of a 16-token span of the packed token axis (lanes
// = consecutive channels, so every load is a contiguous row segment), finds
// the sequence of its first token by binary search in cu_seqlens, preloads
// its 16 inputs and the K-1 before them (from x, or from the state row at a
// sequence start), and walks the span, restarting the window at every
// sequence boundary inside it.  A second kernel, ordered after the first on
// the stream, writes each sequence's new state row, so no thread overwrites
// a state another thread still has to read.
//
// Update (decode): one thread per (row, channel): read the state row, the
// input and the taps, write y and the rolled state.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kSpan = 16;   // tokens per thread in the forward pass
constexpr int kConvXcds = 8;  // accelerator complex dies (separate L2s) on MI355X
#ifndef GDN_CONV_SPAN
#define GDN_CONV_SPAN 8
#endif

// silu(v) = v * sigmoid(v), sigmoid(v) = 1 / (1 + 2^(-v log2 e)), on the
// hardware base-2 exponential and reciprocal (about 1 ulp each; the result
// is within a few ulp of the correctly rounded value).  The library expf and
// an IEEE division cost about 20 instructions per output and made the
// forward pass ALU-bound (195 -> 141 us over 32768 x 5120 fp16).
__device__ __forceinline__ float conv_act(float v, bool silu) {
  return silu ? v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * -1.4426950408889634f))
              : v;
}

// Sequence containing token t: the largest s with cu[s] <= t (zero-length
// sequences share their start with the next one; the last of them wins).
__device__ __forceinline__ int64_t seq_of(const int32_t* cu, int64_t n, int64_t t) {
  int64_t lo = 0, hi = n - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int TX, int K>
__global__ __launch_bounds__(256) void conv_fwd_kernel(ConvArgs a) {
  const int64_t c = (int64_t)blockIdx.y * 256 + threadIdx.x;
  if (c >= a.C) return;
  const int64_t t0 = (int64_t)blockIdx.x * kSpan;
  const int64_t t1 = min(t0 + kSpan, a.T);
  const bool silu = a.silu != 0;

  float w[K];
#pragma unroll
  for (int j = 0; j < K; ++j) w[j] = raw1_to_f32<TX>(load_raw1<TX>(a.w, c * K + j));
  const float bias = a.bias ? raw1_to_f32<TX>(load_raw1<TX>(a.bias, c)) : 0.0f;

  // inputs of the span (clamped to T; the tail is never used)
  float xs[kSpan];
#pragma unroll
  for (int i = 0; i < kSpan; ++i)
    xs[i] = raw1_to_f32<TX>(load_raw1<TX>(a.x, min(t0 + i, a.T - 1) * a.x_rs + c));

  int64_t s = seq_of(a.cu, a.n, t0);
  int64_t s_begin = a.cu[s], s_end = a.cu[s + 1];
  // the window before t0
  float win[K > 1 ? K - 1 : 1];
  bool ok = true;   // the sequence's slot is in range (else all its outputs are NaN)
  auto load_window = [&](int64_t t) {
    // inputs at positions t-(K-1) .. t-1 of sequence s (state or zeros before it)
    const int64_t slot = a.idx ? (int64_t)a.idx[s] : s;
    ok = K == 1 || (slot >= 0 && slot < a.num_slots);   // width 1 keeps no state
    const bool init = ok && (a.has_init ? a.has_init[s] != 0 : true);
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      const int64_t pos = t - (K - 1) + j - s_begin;
      float v = 0.0f;
      // (clamped: a malformed cu_seqlens must not index outside x)
      if (pos >= 0)
        v = raw1_to_f32<TX>(load_raw1<TX>(
            a.x, max((int64_t)0, min(s_begin + pos, a.T - 1)) * a.x_rs + c));
      else if (init)
        v = load1(a.state, a.state_dt,
                  (slot * a.C + c) * a.state_len + max((int64_t)0, (K - 1) + pos));
      win[j] = v;
    }
  };
  load_window(t0);

#pragma unroll
  for (int i = 0; i < kSpan; ++i) {
    const int64_t t = t0 + i;
    if (t < t1) {
      if (t >= s_end && s + 1 < a.n) {   // next sequence(s): skip empty ones
        while (t >= s_end && s + 1 < a.n) { ++s; s_begin = a.cu[s]; s_end = a.cu[s + 1]; }
        load_window(t);
      }
      float acc = bias;
#pragma unroll
      for (int j = 0; j < K - 1; ++j) acc += w[j] * win[j];
      acc += w[K - 1] * xs[i];
      store1(a.out, a.out_dt, t * a.C + c, ok ? conv_act(acc, silu) : __builtin_nanf(""));
#pragma unroll
      for (int j = 0; j + 1 < K - 1; ++j) win[j] = win[j + 1];
      if constexpr (K > 1) win[K - 2] = xs[i];
    }
  }
}

// The same forward pass with 16-byte lanes: each thread owns V consecutive
// channels (V = 8 for 16-bit data, 4 for f32) of an 8-token span, so every
// x load and y store of a wave moves 1 KiB of contiguous row.  Used when the
// channel count, the x row stride and the pointers allow 16-byte access.
// The workgroup is as wide as tiles the channels without idle lanes (256,
// 128 or 64 lanes); spans are dealt to the XCDs in contiguous ranges so the
// K-1 rows before a span come from L2 (measured: x is fetched from HBM once,
// not 11/8 times); a span inside one sequence (all but a few) runs as
// straight-line code.  Rows no other thread reads again, and every output
// row, carry the nontemporal hint (measured 4-5 % faster than plain access).
template <int TX>
struct ConvVec {
  static constexpr int V = TX == kF32 ? 4 : 8;
  static constexpr int EB = TX == kF32 ? 4 : 2;
};

template <int TX>
__device__ __forceinline__ uint4 ld16x(const void* p, int64_t elem) {
  return *reinterpret_cast<const uint4*>(static_cast<const char*>(p) + elem * ConvVec<TX>::EB);
}

// The same 16 bytes with the nontemporal (streaming) hint, for rows no other
// thread reads again.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int TX>
__device__ __forceinline__ uint4 ld16x_stream(const void* p, int64_t elem) {
  const u32x4_t r = __builtin_nontemporal_load(
      reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p) + elem * ConvVec<TX>::EB));
  return make_uint4(r[0], r[1], r[2], r[3]);
}

template <int TX>
__device__ __forceinline__ void widen_v(uint4 u, float* v) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  if constexpr (TX == kF32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = TX == kBF16 ? bf16_to_f32(w[i] & 0xffffu) : f16_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = TX == kBF16 ? bf16_to_f32(w[i] >> 16) : f16_to_f32(w[i] >> 16);
    }
  }
}

template <int TX, int K, bool OF32>
__global__ __launch_bounds__(256) void conv_fwd_vec_kernel(ConvArgs a) {
  constexpr int V = ConvVec<TX>::V;
  constexpr int SPAN = GDN_CONV_SPAN;
  // Workgroups are dealt round-robin to the 8 XCDs (each with its own L2).
  // Block b works on logical unit (b % 8) * per + b / 8, units ordered
  // (span, channel block) with channel blocks fastest, so each XCD walks a
  // contiguous range of spans and the K-1 rows a span reads before its first
  // token are still in that XCD's L2 from the span before.
  const int64_t ncb = (a.C / V + blockDim.x - 1) / blockDim.x;
  const int64_t units = (a.T + SPAN - 1) / SPAN * ncb;
  const int64_t per = (units + kConvXcds - 1) / kConvXcds;
  const int64_t unit = (int64_t)(blockIdx.x % kConvXcds) * per + blockIdx.x / kConvXcds;
  if (unit >= units) return;
  const int64_t cb = unit % ncb;
  const int64_t c0 = (cb * blockDim.x + threadIdx.x) * V;
  if (c0 >= a.C) return;
  const int64_t t0 = (unit / ncb) * SPAN;
  const int64_t t1 = min(t0 + SPAN, a.T);
  const bool silu = a.silu != 0;

  // The last K-1 rows of the span are read again as the next span's window
  // (from L2); the rows before them stream past the caches.
  uint4 xr[SPAN];
#pragma unroll
  for (int i = 0; i < SPAN; ++i) {
    const int64_t e = min(t0 + i, a.T - 1) * a.x_rs + c0;
    xr[i] = i < SPAN - (K - 1) ? ld16x_stream<TX>(a.x, e) : ld16x<TX>(a.x, e);
  }
  // taps of the V channels: V*K contiguous elements, K 16-byte chunks
  float wf[V * K];
#pragma unroll
  for (int i = 0; i < K; ++i) widen_v<TX>(ld16x<TX>(a.w, c0 * K + i * V), wf + i * V);
  float bias[V];
  if (a.bias) {
    widen_v<TX>(ld16x<TX>(a.bias, c0), bias);
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) bias[v] = 0.0f;
  }

  int64_t s = seq_of(a.cu, a.n, t0);
  int64_t s_begin = a.cu[s], s_end = a.cu[s + 1];
  float win[K > 1 ? K - 1 : 1][V];
  bool ok = true;   // the sequence's slot is in range (else all its outputs are NaN)
  auto load_window = [&](int64_t t) {
    const int64_t slot = a.idx ? (int64_t)a.idx[s] : s;
    ok = K == 1 || (slot >= 0 && slot < a.num_slots);   // width 1 keeps no state
    const bool init = ok && (a.has_init ? a.has_init[s] != 0 : true);
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      const int64_t pos = t - (K - 1) + j - s_begin;
      if (pos >= 0) {
        widen_v<TX>(ld16x<TX>(a.x, max((int64_t)0, min(s_begin + pos, a.T - 1)) * a.x_rs + c0),
                    win[j]);
      } else {
#pragma unroll
        for (int v = 0; v < V; ++v)
          win[j][v] = init ? load1(a.state, a.state_dt,
                                   ((slot * a.C + c0 + v) * a.state_len) +
                                       max((int64_t)0, (K - 1) + pos))
                           : 0.0f;
      }
    }
  };
  load_window(t0);

  // one output row: y = act(bias + taps . (window, x_t)), then shift the window
  auto emit = [&](int64_t t, const uint4& xraw) {
    float xv[V], y[V];
    widen_v<TX>(xraw, xv);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float acc = bias[v];
#pragma unroll
      for (int j = 0; j < K - 1; ++j) acc += wf[v * K + j] * win[j][v];
      acc += wf[v * K + K - 1] * xv[v];
      y[v] = ok ? conv_act(acc, silu) : __builtin_nanf("");
    }
    // output rows are written once and not read back: streaming stores
    if constexpr (OF32 || TX == kF32) {
      float* o = static_cast<float*>(a.out) + t * a.C + c0;
#pragma unroll
      for (int q = 0; q < V / 4; ++q) {
        const f32x4_t r = {y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]};
        __builtin_nontemporal_store(r, reinterpret_cast<f32x4_t*>(o + 4 * q));
      }
    } else {
      uint32_t pk[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        pk[q] = TX == kBF16 ? pack2_bf16(y[2 * q], y[2 * q + 1]) : pack2_f16(y[2 * q], y[2 * q + 1]);
      const u32x4_t r = {pk[0], pk[1], pk[2], pk[3]};
      __builtin_nontemporal_store(
          r, reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.out) + t * a.C + c0));
    }
#pragma unroll
    for (int j = 0; j + 1 < K - 1; ++j)
#pragma unroll
      for (int v = 0; v < V; ++v) win[j][v] = win[j + 1][v];
    if constexpr (K > 1) {
#pragma unroll
      for (int v = 0; v < V; ++v) win[K - 2][v] = xv[v];
    }
  };

  if (t1 == t0 + SPAN && t1 <= s_end) {
    // the whole span inside one sequence (all but a few spans): straight-line code
#pragma unroll
    for (int i = 0; i < SPAN; ++i) emit(t0 + i, xr[i]);
    return;
  }
#pragma unroll
  for (int i = 0; i < SPAN; ++i) {
    const int64_t t = t0 + i;
    if (t < t1) {
      if (t >= s_end && s + 1 < a.n) {
        while (t >= s_end && s + 1 < a.n) { ++s; s_begin = a.cu[s]; s_end = a.cu[s + 1]; }
        load_window(t);
      }
      emit(t, xr[i]);
    }
  }
}

// New state rows: the last K-1 entries of (initial window, the inputs).
__global__ __launch_bounds__(256) void conv_state_kernel(ConvArgs a) {
  const int64_t c = (int64_t)blockIdx.y * 256 + threadIdx.x;
  const int64_t s = blockIdx.x;
  if (c >= a.C) return;
  const int64_t slot = a.idx ? (int64_t)a.idx[s] : s;
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t b0 = max((int64_t)0, min((int64_t)a.cu[s], a.T));
  const int64_t len = max((int64_t)0, min((int64_t)a.cu[s + 1], a.T) - b0);
  const bool init = a.has_init ? a.has_init[s] != 0 : true;
  const int64_t row = (slot * a.C + c) * a.state_len;
  const int km1 = a.K - 1;
  float nv[7];
  for (int j = 0; j < km1; ++j) {
    const int64_t e = len + j;   // index into (window of K-1 | inputs)
    nv[j] = e >= km1 ? load1(a.x, a.x_dt, (b0 + e - km1) * a.x_rs + c)
                     : (init ? load1(a.state, a.state_dt, row + e) : 0.0f);
  }
  for (int j = 0; j < km1; ++j) store1(a.state, a.state_dt, row + j, nv[j]);
}

template <int TX, int K>
__global__ __launch_bounds__(256) void conv_update_kernel(ConvArgs a) {
  const int64_t c = (int64_t)blockIdx.y * 256 + threadIdx.x;
  const int64_t r = blockIdx.x;
  if (c >= a.C) return;
  const int64_t slot = a.idx ? (int64_t)a.idx[r] : r;
  if (slot < 0) return;                     // padded row: output and state untouched
  if (K > 1 && slot >= a.num_slots) {       // caller error: NaN, no state access
    store1(a.out, a.out_dt, r * a.C + c, __builtin_nanf(""));
    return;
  }
  const int64_t row = (slot * a.C + c) * a.state_len;
  float st[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) st[j] = load1(a.state, a.state_dt, row + j);
  const float xv = raw1_to_f32<TX>(load_raw1<TX>(a.x, r * a.x_rs + c));
  float acc = a.bias ? raw1_to_f32<TX>(load_raw1<TX>(a.bias, c)) : 0.0f;
#pragma unroll
  for (int j = 0; j < K - 1; ++j) acc += raw1_to_f32<TX>(load_raw1<TX>(a.w, c * K + j)) * st[j];
  acc += raw1_to_f32<TX>(load_raw1<TX>(a.w, c * K + K - 1)) * xv;
  store1(a.out, a.out_dt, r * a.C + c, conv_act(acc, a.silu != 0));
#pragma unroll
  for (int j = 0; j + 1 < K - 1; ++j) store1(a.state, a.state_dt, row + j, st[j + 1]);
  if constexpr (K > 1) store1(a.state, a.state_dt, row + K - 2, xv);
}

template <int TX, bool OF32>
hipError_t launch_fwd_vec(const ConvArgs& a, hipStream_t stream) {
  constexpr int V = ConvVec<TX>::V;
  // the workgroup width (in lanes of V channels) that tiles the channels
  // without idle lanes where one does
  const int64_t lanes = a.C / V;
  const unsigned nthr = lanes % 256 == 0 ? 256 : lanes % 128 == 0 ? 128 : lanes % 64 == 0 ? 64 : 256;
  const int64_t units = (a.T + GDN_CONV_SPAN - 1) / GDN_CONV_SPAN * ((lanes + nthr - 1) / nthr);
  const int64_t blocks = (units + kConvXcds - 1) / kConvXcds * kConvXcds;
  if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  switch (a.K) {
#define GDN_CONV_K(KK) \
    case KK: \
      hipLaunchKernelGGL((conv_fwd_vec_kernel<TX, KK, OF32>), grid, dim3(nthr), 0, stream, a); \
      break;
    GDN_CONV_K(1) GDN_CONV_K(2) GDN_CONV_K(3) GDN_CONV_K(4) GDN_CONV_K(5) GDN_CONV_K(6)
    GDN_CONV_K(7) GDN_CONV_K(8)
#undef GDN_CONV_K
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// 16-byte lanes need V-aligned channel counts, x rows and pointers.
bool conv_vec_ok(const ConvArgs& a) {
  const int v = a.x_dt == kF32 ? 4 : 8;
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) % 16) == 0; };
  return a.C % v == 0 && a.x_rs % v == 0 && al(a.x) && al(a.w) && al(a.bias) && al(a.out) &&
         (a.out_dt == kF32 || a.out_dt == a.x_dt);
}

template <int TX>
hipError_t launch_fwd_tx(const ConvArgs& a, hipStream_t stream) {
  if (conv_vec_ok(a))
    return a.out_dt == kF32 ? launch_fwd_vec<TX, true>(a, stream)
                            : launch_fwd_vec<TX, false>(a, stream);
  const dim3 grid((unsigned)((a.T + kSpan - 1) / kSpan), (unsigned)((a.C + 255) / 256));
  switch (a.K) {
#define GDN_CONV_K(KK) \
    case KK: hipLaunchKernelGGL((conv_fwd_kernel<TX, KK>), grid, dim3(256), 0, stream, a); break;
    GDN_CONV_K(1) GDN_CONV_K(2) GDN_CONV_K(3) GDN_CONV_K(4) GDN_CONV_K(5) GDN_CONV_K(6)
    GDN_CONV_K(7) GDN_CONV_K(8)
#undef GDN_CONV_K
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The update with 16-byte lanes (16-bit x, state_len == K-1): each thread
// owns 8 channels of one row, whose state rows are 8(K-1) contiguous
// elements, read and written back as whole 16-byte chunks; x, the taps and
// the output move 16 bytes per lane as in the forward pass.
template <int TX, int K, int TS>
__global__ __launch_bounds__(256) void conv_update_vec_kernel(ConvArgs a) {
  constexpr int V = ConvVec<TX>::V;
  static_assert(V == 8 && K >= 2, "16-bit inputs, width >= 2");
  constexpr int ES = TS == kF32 ? 4 : 2;
  constexpr int NS = V * (K - 1);          // state elements of the thread's channels
  constexpr int NQ = NS * ES / 16;         // 16-byte chunks of them
  const int64_t c0 = ((int64_t)blockIdx.y * blockDim.x + threadIdx.x) * V;
  const int64_t r = blockIdx.x;
  if (c0 >= a.C) return;
  const int64_t slot = a.idx ? (int64_t)a.idx[r] : r;
  if (slot < 0) return;                     // padded row: output and state untouched
  const bool of32 = a.out_dt == kF32;
  if (slot >= a.num_slots) {                // caller error: NaN, no state access
    for (int v = 0; v < V; ++v) store1(a.out, a.out_dt, r * a.C + c0 + v, __builtin_nanf(""));
    return;
  }
  uint4* sp = reinterpret_cast<uint4*>(static_cast<char*>(a.state) +
                                       (slot * a.C + c0) * (int64_t)(K - 1) * ES);
  uint4 sq[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) sq[i] = sp[i];
  float xv[V], wf[V * K], st[NS];
  widen_v<TX>(ld16x<TX>(a.x, r * a.x_rs + c0), xv);
#pragma unroll
  for (int i = 0; i < K; ++i) widen_v<TX>(ld16x<TX>(a.w, c0 * K + i * V), wf + i * V);
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    if constexpr (TS == kF32) widen_v<kF32>(sq[i], st + 4 * i);
    else widen_v<TS>(sq[i], st + 8 * i);
  }
  float bias[V];
  if (a.bias) {
    widen_v<TX>(ld16x<TX>(a.bias, c0), bias);
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) bias[v] = 0.0f;
  }
  const bool silu = a.silu != 0;
  float y[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float acc = bias[v];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) acc += wf[v * K + j] * st[v * (K - 1) + j];
    acc += wf[v * K + K - 1] * xv[v];
    y[v] = conv_act(acc, silu);
  }
  if (of32) {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(a.out) + r * a.C + c0);
    o[0] = make_float4(y[0], y[1], y[2], y[3]);
    o[1] = make_float4(y[4], y[5], y[6], y[7]);
  } else {
    uint32_t pk[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      pk[q] = TX == kBF16 ? pack2_bf16(y[2 * q], y[2 * q + 1]) : pack2_f16(y[2 * q], y[2 * q + 1]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + r * a.C + c0) =
        make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
  // rolled rows: the last K-2 entries move up, the input enters at the end
  float ns[NS];
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int j = 0; j + 1 < K - 1; ++j) ns[v * (K - 1) + j] = st[v * (K - 1) + j + 1];
    ns[v * (K - 1) + K - 2] = xv[v];
  }
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    uint4 q;
    if constexpr (TS == kF32) {
      q = make_uint4(__float_as_uint(ns[4 * i]), __float_as_uint(ns[4 * i + 1]),
                     __float_as_uint(ns[4 * i + 2]), __float_as_uint(ns[4 * i + 3]));
    } else {
      const float* e = ns + 8 * i;
      auto p2 = [](float lo, float hi) {
        return TS == kBF16 ? pack2_bf16(lo, hi) : pack2_f16(lo, hi);
      };
      q = make_uint4(p2(e[0], e[1]), p2(e[2], e[3]), p2(e[4], e[5]), p2(e[6], e[7]));
    }
    sp[i] = q;
  }
}

// The 16-byte update applies when x is 16-bit, the width is 2..5, the state
// rows hold exactly K-1 entries, the channels and x's row stride are
// multiples of 8 and every buffer is 16-byte aligned.
template <int TX>
static bool update_vec_ok(const ConvArgs& a) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) % 16) == 0; };
  return TX != kF32 && a.K >= 2 && a.K <= 5 && a.state_len == a.K - 1 && a.C % 8 == 0 &&
         a.x_rs % 8 == 0 && al(a.x) && al(a.w) && (a.bias == nullptr || al(a.bias)) &&
         al(a.out) && al(a.state);
}

template <int TX, int TS>
hipError_t launch_update_vec(const ConvArgs& a, hipStream_t stream) {
  const int64_t lanes = a.C / 8;
  const unsigned nthr = lanes >= 256 ? 256 : lanes >= 128 ? 128 : 64;
  const dim3 grid((unsigned)a.n, (unsigned)((lanes + nthr - 1) / nthr));
  switch (a.K) {
#define GDN_CONV_K(KK) \
    case KK: \
      hipLaunchKernelGGL((conv_update_vec_kernel<TX, KK, TS>), grid, dim3(nthr), 0, stream, a); \
      break;
    GDN_CONV_K(2) GDN_CONV_K(3) GDN_CONV_K(4) GDN_CONV_K(5)
#undef GDN_CONV_K
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int TX>
hipError_t launch_update_tx(const ConvArgs& a, hipStream_t stream) {
  if constexpr (TX != kF32) {
    if (update_vec_ok<TX>(a)) {
      return a.state_dt == kF32  ? launch_update_vec<TX, kF32>(a, stream)
           : a.state_dt == kBF16 ? launch_update_vec<TX, kBF16>(a, stream)
                                 : launch_update_vec<TX, kF16>(a, stream);
    }
  }
  const dim3 grid((unsigned)a.n, (unsigned)((a.C + 255) / 256));
  switch (a.K) {
#define GDN_CONV_K(KK) \
    case KK: hipLaunchKernelGGL((conv_update_kernel<TX, KK>), grid, dim3(256), 0, stream, a); break;
    GDN_CONV_K(1) GDN_CONV_K(2) GDN_CONV_K(3) GDN_CONV_K(4) GDN_CONV_K(5) GDN_CONV_K(6)
    GDN_CONV_K(7) GDN_CONV_K(8)
#undef GDN_CONV_K
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  if (a.T > 0) {
    hipError_t e = a.x_dt == kBF16 ? launch_fwd_tx<kBF16>(a, stream)
                 : a.x_dt == kF16  ? launch_fwd_tx<kF16>(a, stream)
                                   : launch_fwd_tx<kF32>(a, stream);
    if (e != hipSuccess) return e;
  }
  if (a.K > 1) {
    const dim3 grid((unsigned)a.n, (unsigned)((a.C + 255) / 256));
    hipLaunchKernelGGL(conv_state_kernel, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_conv_update(const ConvArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  return a.x_dt == kBF16 ? launch_update_tx<kBF16>(a, stream)
       : a.x_dt == kF16  ? launch_update_tx<kF16>(a, stream)
                         : launch_update_tx<kF32>(a, stream);
}

}  // namespace gdn
