// gdn_chunked.hip -- chunk-parallel varlen prefill with the dense products on
// MFMA (v_mfma_f32_16x16x32_{bf16,f16}), for Dk = 128, Dv a multiple of 32 and
// bf16 / fp16 inputs.
//
// The recurrence (vllm.cpp tests/vt/test_ops_gdn.cpp, "gdn decode:
// hand-computed single step"), per v-head with k, q already normalised and q
// scaled:  S_t = d_t S_{t-1} + u_t k_t^T,  u_t = beta_t (v_t - d_t S_{t-1} k_t),
// o_t = S_t q_t.  Over a chunk of C tokens with entry state S0, cumulative
// log-decay G_i = sum_{j<=i} g_j and E_ij = exp(G_i - G_j) (j <= i), the same
// recurrence unrolls to (rows are tokens):
//   (I + A) U = diag(beta) (V - diag(e^G) K S0^T),  A_ij = beta_i E_ij k_i.k_j (j < i)
//   O   = diag(e^G) Q S0^T + (E o Q K^T) U           (E including the diagonal)
//   S_C = e^{G_C} S0 + U^T diag(e^{G_C - G}) K
// This is only a reassociation of the token loop; no step is approximated.
//
// Work split:
//   chunk_meta_kernel   prefix count of chunks per sequence, from cu_seqlens on
//                       the device (no host synchronisation);
//   chunk_t_kernel      one workgroup per (chunk, v-head): K K^T on MFMA, the
//                       strictly-lower A, T = (I + A)^{-1} by blocked forward
//                       substitution (16x16 blocks), T_b = T diag(beta) to the
//                       workspace -- all of it independent of the state;
//   chunk_state_kernel  one workgroup per (sequence, v-head, 32-row tile of S)
//                       walks the chunks in order with its S tile held in MFMA
//                       accumulators:
//                         X = K S^T,  Z = V - diag(e^G n_k) X,  U = T_b Z,
//                         O = diag(e^G scale n_q) Q S^T + P U,
//                         S = e^{G_C} S + (diag(e^{G_C - G} n_k) U)^T K.
//                       Forming U as T_b (V - ...) never builds the 64 x 128
//                       matrix T diag(beta e^G) K, so each tile does only work
//                       proportional to its own 32 rows.
// Precision: the raw 16-bit q/k/v are exact MFMA operands; the L2 norms enter
// as diagonal scalings; an f32 operand (S, T_b, Z, U) is split into a 16-bit
// high part and a 16-bit remainder, and the products keep hi*hi + hi*lo +
// lo*hi (both sides computed) or hi + lo (one side raw), which carries about
// 16 significant bits -- the state is accumulated in f32 throughout.  The
// cumulative gate G is summed in f64 so differences G_i - G_j stay exact even
// when a head's gate is thousands per chunk.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int CK = 64;        // tokens per chunk
constexpr int DKC = 128;      // key head size served here
constexpr int BVT = 32;       // state rows per workgroup in the state walk
constexpr int LDQ = DKC + 8;  // padded LDS row (16-bit elements), token-major 128-wide tiles
constexpr int LDT = CK + 8;   // padded LDS row (16-bit elements), 64-wide tiles
constexpr int LDF = CK + 4;   // padded LDS row (f32), 64 x 64 matrices

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int TIN>
struct MT;

template <>
struct MT<kBF16> {
  typedef __bf16 x8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x4 mma(x8 a, x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t enc(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  }
  static __device__ __forceinline__ float dec(uint32_t u) { return bf16_to_f32(u); }
};

template <>
struct MT<kF16> {
  typedef _Float16 x8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x4 mma(x8 a, x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t enc(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  static __device__ __forceinline__ float dec(uint32_t u) { return f16_to_f32(u); }
};

// MFMA operand (16 rows x 32 k) from a row-major 16-bit LDS matrix: lane l
// takes row r0 + l%16, elements k0 + 8 (l/16) .. +8.  Serves both the A
// operand (rows = M) and the B operand stored transposed (rows = N).
template <int TIN>
__device__ __forceinline__ typename MT<TIN>::x8 frag(const uint16_t* m, int ld, int r0, int k0,
                                                     int lane) {
  return *reinterpret_cast<const typename MT<TIN>::x8*>(m + (r0 + (lane & 15)) * ld + k0 +
                                                        8 * (lane >> 4));
}

// The same operand from an f32 LDS matrix, split into high and low 16-bit parts.
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

template <int TIN>
__device__ __forceinline__ void frag_split(const float* m, int ld, int r0, int k0, int lane,
                                           typename MT<TIN>::x8& hi, typename MT<TIN>::x8& lo) {
  const float* p = m + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4);
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  u16x8 h, l;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = MT<TIN>::enc(x[e]);
    l[e] = MT<TIN>::enc(x[e] - MT<TIN>::dec(h[e]));
  }
  hi = __builtin_bit_cast(typename MT<TIN>::x8, h);
  lo = __builtin_bit_cast(typename MT<TIN>::x8, l);
}

__device__ __forceinline__ void chunk_bounds(const PrefillArgs& a, int64_t s, int64_t& t0,
                                             int64_t& t1) {
  // cu_seqlens is device data: clamp so a malformed table cannot index past
  // the token arrays.
  t1 = min((int64_t)a.cu[s + 1], a.total_tokens);
  t0 = max((int64_t)0, min((int64_t)a.cu[s], t1));
}

// ---------------------------------------------------------------------------
// chunk offsets: cs[s] = number of chunks of sequences before s; cs[n] = total
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void chunk_meta_kernel(PrefillArgs a, int32_t* cs) {
  __shared__ int32_t part[256];
  int32_t carry = 0;
  if (threadIdx.x == 0) cs[0] = 0;
  for (int64_t base = 0; base < a.num_seqs; base += 256) {
    const int64_t s = base + threadIdx.x;
    int32_t c = 0;
    if (s < a.num_seqs) {
      int64_t t0, t1;
      chunk_bounds(a, s, t0, t1);
      c = (int32_t)((t1 - t0 + CK - 1) / CK);
    }
    part[threadIdx.x] = c;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int32_t add = threadIdx.x >= (unsigned)off ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += add;
      __syncthreads();
    }
    if (s < a.num_seqs) cs[s + 1] = carry + part[threadIdx.x];
    carry += part[255];
    __syncthreads();
  }
}

// inclusive prefix sum of 64 values held one per lane of a wave, in f64
__device__ __forceinline__ double wave_prefix64(double x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// ---------------------------------------------------------------------------
// T_b = (I + A)^{-1} diag(beta) per (chunk, v-head)
// ---------------------------------------------------------------------------
template <int TIN>
__global__ __launch_bounds__(256) void chunk_t_kernel(PrefillArgs a, const int32_t* cs,
                                                      float* tws) {
  __shared__ __align__(16) uint16_t Ks[CK * LDQ];
  __shared__ __align__(16) float Am[CK * LDF];
  __shared__ __align__(16) float Tm[CK * LDF];
  __shared__ float Rs[4][16 * 17];
  __shared__ double Gd[CK];
  __shared__ float nk[CK];
  __shared__ float bt[CK];

  const int c = blockIdx.x;
  const int h = blockIdx.y;
  const int n = (int)a.num_seqs;
  if (c >= cs[n]) return;
  int lo = 0, hi = n - 1;  // largest s with cs[s] <= c
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cs[mid] <= c) lo = mid; else hi = mid - 1;
  }
  const int s = lo;
  int64_t t0, t1;
  chunk_bounds(a, s, t0, t1);
  const int64_t tb = t0 + (int64_t)(c - cs[s]) * CK;
  const int L = (int)min((int64_t)CK, t1 - tb);
  const int hk = h / (a.hv / a.hk);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // stage K (zero rows past the sequence), g, beta
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = tid + 256 * u;
    const int row = idx >> 4, p = idx & 15;
    uint4 val = {0, 0, 0, 0};
    if (row < L)
      val = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) +
                                            (tb + row) * a.k_rs + (int64_t)hk * DKC + 8 * p);
    *reinterpret_cast<uint4*>(Ks + row * LDQ + 8 * p) = val;
  }
  if (w == 0) {
    const float gv = lane < L ? a.g[(tb + lane) * a.g_rs + h] : 0.0f;
    const float bv = lane < L ? a.beta[(tb + lane) * a.beta_rs + h] : 0.0f;
    Gd[lane] = wave_prefix64((double)gv, lane);
    bt[lane] = bv;
  }
  __syncthreads();
  {  // row norms of K: 4 lanes per row
    const int row = tid >> 2, qq = tid & 3;
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float x = MT<TIN>::dec(Ks[row * LDQ + 32 * qq + e]);
      ss += x * x;
    }
    ss += xor_lane<1>(ss);
    ss += xor_lane<2>(ss);
    if (qq == 0) nk[row] = a.l2norm ? 1.0f / sqrtf(ss + a.l2_eps) : 1.0f;
  }
  __syncthreads();

  // A = strictly lower (beta_i E_ij nk_i nk_j (K K^T)_ij), lower tiles only
  for (int t = w; t < 10; t += 4) {
    const int ti = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
    const int tj = t - (ti * (ti + 1)) / 2;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      acc = MT<TIN>::mma(frag<TIN>(Ks, LDQ, 16 * ti, 32 * kk, lane),
                         frag<TIN>(Ks, LDQ, 16 * tj, 32 * kk, lane), acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * (lane >> 4) + r;
      const int j = 16 * tj + (lane & 15);
      float v = 0.0f;
      if (j < i) v = bt[i] * expf((float)(Gd[i] - Gd[j])) * nk[i] * nk[j] * acc[r];
      Am[i * LDF + j] = v;
    }
  }
  // zero the strictly-upper 16x16 blocks of T
  for (int idx = tid; idx < 6 * 256; idx += 256) {
    const int blk = idx >> 8, e = idx & 255;
    const int bi = blk < 3 ? 0 : blk < 5 ? 1 : 2;
    const int bj = blk < 3 ? blk + 1 : blk < 5 ? blk - 1 : 3;
    Tm[(16 * bi + (e >> 4)) * LDF + 16 * bj + (e & 15)] = 0.0f;
  }
  __syncthreads();

  // diagonal blocks: forward substitution, one column per lane
  if (lane < 16) {
    const int b0 = 16 * w, col = lane;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = (r == col) ? 1.0f : 0.0f;
#pragma unroll
      for (int m = 0; m < r; ++m) v -= Am[(b0 + r) * LDF + b0 + m] * x[m];
      x[r] = v;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tm[(b0 + r) * LDF + b0 + col] = x[r];
  }
  __syncthreads();

  // off-diagonal blocks by distance: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
  for (int d = 1; d < 4; ++d) {
    const int j = w, i = w + d;
    const bool active = i < 4;
    const int cc = lane & 15, rb = 4 * (lane >> 4);
    if (active) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = rb + q;
        float r = 0.0f;
        for (int k = j; k < i; ++k)
#pragma unroll
          for (int m = 0; m < 16; ++m)
            r += Am[(16 * i + rr) * LDF + 16 * k + m] * Tm[(16 * k + m) * LDF + 16 * j + cc];
        Rs[w][rr * 17 + cc] = r;
      }
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = rb + q;
        float t = 0.0f;
#pragma unroll
        for (int m = 0; m < 16; ++m) t += Tm[(16 * i + rr) * LDF + 16 * i + m] * Rs[w][m * 17 + cc];
        Tm[(16 * i + rr) * LDF + 16 * j + cc] = -t;
      }
    }
    __syncthreads();
  }

  float* out = tws + ((int64_t)c * a.hv + h) * (CK * CK);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = tid + 256 * u;
    const int i = idx >> 4, j4 = 4 * (idx & 15);
    float4 t = *reinterpret_cast<const float4*>(Tm + i * LDF + j4);
    t.x *= bt[j4]; t.y *= bt[j4 + 1]; t.z *= bt[j4 + 2]; t.w *= bt[j4 + 3];
    *reinterpret_cast<float4*>(out + i * CK + j4) = t;
  }
}

// ---------------------------------------------------------------------------
// the state walk
// ---------------------------------------------------------------------------
template <int TIN>
struct WalkLds {
  uint16_t Qs[CK * LDQ];
  uint16_t Ks[CK * LDQ];
  uint16_t Kt[DKC * LDT];
  uint16_t Vs[CK * BVT];
  float Ts[CK * LDF];
  uint16_t Sh[BVT * LDQ], Sl[BVT * LDQ];
  uint16_t Zh[BVT * LDT], Zl[BVT * LDT];
  uint16_t Uh[BVT * LDT], Ul[BVT * LDT];
  uint16_t Wh[BVT * LDT], Wl[BVT * LDT];
  uint16_t Ph[CK * LDT];
  double Gd[CK];
  float nq[CK], nk[CK];
};

template <int TIN>
__global__ __launch_bounds__(256) void chunk_state_kernel(PrefillArgs a, const int32_t* cs,
                                                          const float* tws, int ntiles,
                                                          int max_chunks) {
  __shared__ __align__(16) WalkLds<TIN> sm;
  using M = MT<TIN>;
  using x8 = typename M::x8;

  const int tile = blockIdx.x % ntiles;
  const int sh = blockIdx.x / ntiles;
  const int h = sh % a.hv;
  const int s = sh / a.hv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dv0 = tile * BVT;
  const int hk = h / (a.hv / a.hk);
  int64_t t_begin, t_end;
  chunk_bounds(a, s, t_begin, t_end);
  const int c0 = cs[s];
  // a well-formed cu_seqlens gives c0 + nch <= max_chunks; a malformed one
  // (overlapping ranges) must still never index past the workspace
  const int nch = max(0, min((int)((t_end - t_begin + CK - 1) / CK), max_chunks - c0));
  const int64_t slot = a.idx ? (int64_t)a.idx[s] : (int64_t)s;
  const int64_t out_rs = (int64_t)a.hv * a.dv;

  if (slot < 0 || slot >= a.num_slots) {
    // caller error: NaN outputs for this tile, no state access
    for (int64_t t = t_begin + (tid >> 3); t < t_end; t += 32)
      for (int e = (tid & 7); e < BVT; e += 8)
        store1(a.out, a.out_dt, t * out_rs + (int64_t)h * a.dv + dv0 + e, __builtin_nanf(""));
    return;
  }
  const bool init = a.has_init ? a.has_init[s] != 0 : true;
  float* Sg = a.pool + ((slot * a.hv + h) * a.dv + dv0) * DKC;

  // S tile in MFMA accumulators: wave w holds (mt, nt) = (q / 2, 2w + q % 2);
  // element r of tile q is S[16 mt + 4 (lane/16) + r][16 nt + lane % 16].
  f32x4 accs[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int mt = q >> 1, nt = 2 * w + (q & 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * mt + 4 * (lane >> 4) + r, col = 16 * nt + (lane & 15);
      accs[q][r] = init ? Sg[row * DKC + col] : 0.0f;
    }
  }
  auto write_s_lds = [&]() {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int mt = q >> 1, nt = 2 * w + (q & 1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * mt + 4 * (lane >> 4) + r, col = 16 * nt + (lane & 15);
        const uint16_t hb = M::enc(accs[q][r]);
        sm.Sh[row * LDQ + col] = hb;
        sm.Sl[row * LDQ + col] = M::enc(accs[q][r] - M::dec(hb));
      }
    }
  };
  write_s_lds();

  for (int ch = 0; ch < nch; ++ch) {
    const int64_t tb = t_begin + (int64_t)ch * CK;
    const int L = (int)min((int64_t)CK, t_end - tb);
    // ---- stage the chunk's inputs ----
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = tid + 256 * u;
      const int row = idx >> 4, p = idx & 15;
      uint4 qv = {0, 0, 0, 0}, kv = {0, 0, 0, 0};
      if (row < L) {
        qv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) +
                                             (tb + row) * a.q_rs + (int64_t)hk * DKC + 8 * p);
        kv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) +
                                             (tb + row) * a.k_rs + (int64_t)hk * DKC + 8 * p);
      }
      *reinterpret_cast<uint4*>(sm.Qs + row * LDQ + 8 * p) = qv;
      *reinterpret_cast<uint4*>(sm.Ks + row * LDQ + 8 * p) = kv;
      const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.Kt[(8 * p + 2 * e) * LDT + row] = (uint16_t)(kw[e] & 0xffffu);
        sm.Kt[(8 * p + 2 * e + 1) * LDT + row] = (uint16_t)(kw[e] >> 16);
      }
    }
    {
      const int row = tid >> 2, p = tid & 3;
      uint4 vv = {0, 0, 0, 0};
      if (row < L)
        vv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v) +
                                             (tb + row) * a.v_rs + (int64_t)h * a.dv + dv0 + 8 * p);
      *reinterpret_cast<uint4*>(sm.Vs + row * BVT + 8 * p) = vv;
    }
    {
      const float* tsrc = tws + ((int64_t)(c0 + ch) * a.hv + h) * (CK * CK);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = tid + 256 * u;
        const int i = idx >> 4, j4 = 4 * (idx & 15);
        *reinterpret_cast<float4*>(sm.Ts + i * LDF + j4) =
            *reinterpret_cast<const float4*>(tsrc + i * CK + j4);
      }
    }
    if (w == 0) {
      const float gv = lane < L ? a.g[(tb + lane) * a.g_rs + h] : 0.0f;
      sm.Gd[lane] = wave_prefix64((double)gv, lane);
    }
    __syncthreads();
    {  // row norms of q and k
      const int row = tid >> 2, qq = tid & 3;
      float sq = 0.0f, sk = 0.0f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float x = M::dec(sm.Qs[row * LDQ + 32 * qq + e]);
        const float y = M::dec(sm.Ks[row * LDQ + 32 * qq + e]);
        sq += x * x;
        sk += y * y;
      }
      sq += xor_lane<1>(sq);
      sq += xor_lane<2>(sq);
      sk += xor_lane<1>(sk);
      sk += xor_lane<2>(sk);
      if (qq == 0) {
        sm.nq[row] = a.l2norm ? 1.0f / sqrtf(sq + a.l2_eps) : 1.0f;
        sm.nk[row] = a.l2norm ? 1.0f / sqrtf(sk + a.l2_eps) : 1.0f;
      }
    }
    __syncthreads();

    // ---- phase 1: P (row block w), X = K S^T and Q S^T (rows 16w.., both column tiles) ----
    const int rb = 16 * w;
    {
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (tj <= w) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            acc = M::mma(frag<TIN>(sm.Qs, LDQ, rb, 32 * kk, lane),
                         frag<TIN>(sm.Ks, LDQ, 16 * tj, 32 * kk, lane), acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = rb + 4 * (lane >> 4) + r;
          const int j = 16 * tj + (lane & 15);
          float p = 0.0f;
          if (j <= i)
            p = acc[r] * a.scale * sm.nq[i] * sm.nk[j] * expf((float)(sm.Gd[i] - sm.Gd[j]));
          sm.Ph[i * LDT + j] = M::enc(p);
        }
      }
    }
    f32x4 accq[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 accx = {0.f, 0.f, 0.f, 0.f};
      accq[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const x8 shi = frag<TIN>(sm.Sh, LDQ, 16 * nt, 32 * kk, lane);
        const x8 slo = frag<TIN>(sm.Sl, LDQ, 16 * nt, 32 * kk, lane);
        const x8 kf = frag<TIN>(sm.Ks, LDQ, rb, 32 * kk, lane);
        const x8 qf = frag<TIN>(sm.Qs, LDQ, rb, 32 * kk, lane);
        accx = M::mma(kf, shi, accx);
        accx = M::mma(kf, slo, accx);
        accq[nt] = M::mma(qf, shi, accq[nt]);
        accq[nt] = M::mma(qf, slo, accq[nt]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = rb + 4 * (lane >> 4) + r;
        const int dvl = 16 * nt + (lane & 15);
        const float z = M::dec(sm.Vs[i * BVT + dvl]) -
                        expf((float)sm.Gd[i]) * sm.nk[i] * accx[r];
        const uint16_t zh = M::enc(z);
        sm.Zh[dvl * LDT + i] = zh;
        sm.Zl[dvl * LDT + i] = M::enc(z - M::dec(zh));
      }
    }
    __syncthreads();

    // ---- phase 2: U = T_b Z (row block w) ----
    const int nkt = (rb + 15) / 32 + 1;  // k-steps over tokens j <= i
    const float gl = (float)sm.Gd[L - 1];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 accu = {0.f, 0.f, 0.f, 0.f};
      for (int kt = 0; kt < nkt; ++kt) {
        x8 th, tl;
        frag_split<TIN>(sm.Ts, LDF, rb, 32 * kt, lane, th, tl);
        const x8 zh = frag<TIN>(sm.Zh, LDT, 16 * nt, 32 * kt, lane);
        const x8 zl = frag<TIN>(sm.Zl, LDT, 16 * nt, 32 * kt, lane);
        accu = M::mma(th, zh, accu);
        accu = M::mma(th, zl, accu);
        accu = M::mma(tl, zh, accu);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = rb + 4 * (lane >> 4) + r;
        const int dvl = 16 * nt + (lane & 15);
        const float u = accu[r];
        const uint16_t uh = M::enc(u);
        sm.Uh[dvl * LDT + i] = uh;
        sm.Ul[dvl * LDT + i] = M::enc(u - M::dec(uh));
        const float up = u * expf(gl - (float)sm.Gd[i]) * sm.nk[i];
        const uint16_t wh = M::enc(up);
        sm.Wh[dvl * LDT + i] = wh;
        sm.Wl[dvl * LDT + i] = M::enc(up - M::dec(wh));
      }
    }
    __syncthreads();

    // ---- phase 3: outputs of row block w; state update of the wave's S tiles ----
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 acco = {0.f, 0.f, 0.f, 0.f};
      for (int kt = 0; kt < nkt; ++kt) {
        const x8 pf = frag<TIN>(sm.Ph, LDT, rb, 32 * kt, lane);
        acco = M::mma(pf, frag<TIN>(sm.Uh, LDT, 16 * nt, 32 * kt, lane), acco);
        acco = M::mma(pf, frag<TIN>(sm.Ul, LDT, 16 * nt, 32 * kt, lane), acco);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = rb + 4 * (lane >> 4) + r;
        const int dvl = 16 * nt + (lane & 15);
        if (i < L) {
          const float o = expf((float)sm.Gd[i]) * a.scale * sm.nq[i] * accq[nt][r] + acco[r];
          store1(a.out, a.out_dt, (tb + i) * out_rs + (int64_t)h * a.dv + dv0 + dvl, o);
        }
      }
    }
    const float gc = expf(gl);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int mt = q >> 1, nt = 2 * w + (q & 1);
      f32x4 acc = accs[q];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] *= gc;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const x8 kf = frag<TIN>(sm.Kt, LDT, 16 * nt, 32 * kt, lane);
        acc = M::mma(frag<TIN>(sm.Wh, LDT, 16 * mt, 32 * kt, lane), kf, acc);
        acc = M::mma(frag<TIN>(sm.Wl, LDT, 16 * mt, 32 * kt, lane), kf, acc);
      }
      accs[q] = acc;
    }
    __syncthreads();
    write_s_lds();
  }

  // final state
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int mt = q >> 1, nt = 2 * w + (q & 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * mt + 4 * (lane >> 4) + r, col = 16 * nt + (lane & 15);
      Sg[row * DKC + col] = accs[q][r];
    }
  }
}

int64_t max_chunks(int64_t total_tokens, int64_t num_seqs) {
  return (total_tokens + CK - 1) / CK + num_seqs;
}

size_t meta_bytes(int64_t num_seqs) { return (size_t)((num_seqs + 1) * 4 + 255) / 256 * 256; }

template <int TIN>
hipError_t launch_chunked_t(const PrefillArgs& a, void* ws, hipStream_t stream) {
  int32_t* cs = static_cast<int32_t*>(ws);
  float* tws = reinterpret_cast<float*>(static_cast<char*>(ws) + meta_bytes(a.num_seqs));
  const int64_t mc = max_chunks(a.total_tokens, a.num_seqs);
  hipLaunchKernelGGL(chunk_meta_kernel, dim3(1), dim3(256), 0, stream, a, cs);
  hipLaunchKernelGGL((chunk_t_kernel<TIN>), dim3((unsigned)mc, (unsigned)a.hv), dim3(256), 0,
                     stream, a, (const int32_t*)cs, tws);
  const int ntiles = a.dv / BVT;
  const int64_t blocks = a.num_seqs * a.hv * ntiles;
  hipLaunchKernelGGL((chunk_state_kernel<TIN>), dim3((unsigned)blocks), dim3(256), 0, stream, a,
                     (const int32_t*)cs, (const float*)tws, ntiles, (int)mc);
  return hipGetLastError();
}

}  // namespace

bool chunked_supported(int in_dt, int out_dt, int dk, int dv) {
  (void)out_dt;
  return (in_dt == kBF16 || in_dt == kF16) && dk == DKC && dv % BVT == 0;
}

bool chunked_layout_ok(const void* q, const void* k, const void* v, int64_t q_rs, int64_t k_rs,
                       int64_t v_rs) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  return al(q) && al(k) && al(v) && q_rs % 8 == 0 && k_rs % 8 == 0 && v_rs % 8 == 0;
}

size_t chunked_workspace_bytes(int64_t total_tokens, int64_t num_seqs, int hv, int dk, int dv) {
  (void)dk; (void)dv;
  return meta_bytes(num_seqs) +
         (size_t)max_chunks(total_tokens, num_seqs) * (size_t)hv * CK * CK * sizeof(float);
}

hipError_t launch_prefill_chunked(const PrefillArgs& a, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  if (ws_bytes < chunked_workspace_bytes(a.total_tokens, a.num_seqs, a.hv, a.dk, a.dv))
    return hipErrorInvalidValue;
  if (a.num_seqs >= (1 << 30) || max_chunks(a.total_tokens, a.num_seqs) >= (1 << 30))
    return hipErrorInvalidValue;
  if (a.in_dt == kBF16) return launch_chunked_t<kBF16>(a, ws, stream);
  if (a.in_dt == kF16) return launch_chunked_t<kF16>(a, ws, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
