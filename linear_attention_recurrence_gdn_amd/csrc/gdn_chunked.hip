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
//   chunk_state_kernel  one workgroup per (sequence, v-head, 16-row tile of S)
//                       walks the chunks in order with its S tile held in MFMA
//                       accumulators:
//                         X = K S^T,  Z = V - diag(e^G n_k) X,  U = T_b Z,
//                         O = diag(e^G scale n_q) Q S^T + P U,
//                         S = e^{G_C} S + (diag(e^{G_C - G} n_k) U)^T K.
//                       Forming U as T_b (V - ...) never builds the 64 x 128
//                       matrix T diag(beta e^G) K, so each tile does only work
//                       proportional to its own 16 rows.
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
#ifndef GDN_WALK_NT
#define GDN_WALK_NT 2
#endif
constexpr int WALK_NT = GDN_WALK_NT;   // 16-row state tiles per workgroup in the state walk
constexpr int BVT = 16 * WALK_NT;     // state rows per workgroup
constexpr int LDQ = DKC + 8;  // padded LDS row (16-bit elements), token-major 128-wide tiles
constexpr int LDT = CK + 8;   // padded LDS row (16-bit elements), 64-wide tiles
constexpr int LDF = CK + 4;   // padded LDS row (f32), 64 x 64 matrices
constexpr int kXcds = 8;      // accelerator complex dies (separate L2s) on MI355X

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

// Workgroup barrier ordering LDS only.  __syncthreads() also waits for every
// outstanding global access, which would force the next chunk's prefetched
// loads to land at the first barrier; all communication between the waves
// here goes through LDS, so the global loads may stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void chunk_bounds(const PrefillArgs& a, int64_t s, int64_t& t0,
                                             int64_t& t1) {
  // cu_seqlens is device data: clamp so a malformed table cannot index past
  // the token arrays.
  t1 = min((int64_t)a.cu[s + 1], a.total_tokens);
  t0 = max((int64_t)0, min((int64_t)a.cu[s], t1));
}

// ---------------------------------------------------------------------------
// chunk offsets: cs[s] = number of chunks of sequences before s; cs[n] = total.
// order[k] = the sequence with the k-th most chunks (ties by index) when
// n <= kOrderMax, else k: the state walk starts the longest sequences first,
// since the longest one bounds the whole prefill.
// ---------------------------------------------------------------------------
constexpr int kOrderMax = 1024;

__global__ __launch_bounds__(256) void chunk_meta_kernel(PrefillArgs a, int32_t* cs,
                                                         int32_t* order) {
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
  __syncthreads();
  const int n = (int)a.num_seqs;
  for (int s = threadIdx.x; s < n; s += 256) {
    int rank = s;
    if (n <= kOrderMax) {
      const int cnt = cs[s + 1] - cs[s];
      rank = 0;
      for (int t = 0; t < n; ++t) {
        const int ct = cs[t + 1] - cs[t];
        rank += (ct > cnt) || (ct == cnt && t < s);
      }
    }
    order[rank] = s;
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
// Per (chunk, v-head) record written by the prep kernel and read by the state
// walk (byte offsets):
//   T_b = (I + A)^{-1} diag(beta), split into 16-bit high / low parts, [64][64] each
//   P   = masked, scaled Q K^T:  P_ij = scale n_q,i n_k,j E_ij (q_i . k_j) for j <= i,
//         16-bit (high part only; it multiplies U in the output term only)
//   F   = f32 [4][64]: fz_i = e^{G_i} n_k,i,  fo_i = e^{G_i} scale n_q,i,
//         fw_i = e^{G_last - G_i} n_k,i,  and F[3][0] = e^{G_last}
// ---------------------------------------------------------------------------
constexpr int REC_TH = 0;
constexpr int REC_TL = CK * CK * 2;
constexpr int REC_P = 2 * CK * CK * 2;
constexpr int REC_F = 3 * CK * CK * 2;
constexpr int REC_BYTES = REC_F + 4 * CK * 4;

template <int TIN>
__global__ __launch_bounds__(256) void chunk_prep_kernel(PrefillArgs a, const int32_t* cs,
                                                         char* recs) {
  __shared__ __align__(16) uint16_t Qs[CK * LDQ];
  __shared__ __align__(16) uint16_t Ks[CK * LDQ];
  __shared__ __align__(16) float Am[CK * LDF];
  __shared__ __align__(16) float Tm[CK * LDF];
  __shared__ float Rs[4][16 * 17];
  __shared__ double Gd[CK];
  __shared__ float nq[CK], nk[CK], bt[CK];
  using M = MT<TIN>;

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
  char* rec = recs + ((int64_t)c * a.hv + h) * REC_BYTES;

  // stage Q and K (zero rows past the sequence), g, beta
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
    *reinterpret_cast<uint4*>(Qs + row * LDQ + 8 * p) = qv;
    *reinterpret_cast<uint4*>(Ks + row * LDQ + 8 * p) = kv;
  }
  if (w == 0) {
    const float gv = lane < L ? a.g[(tb + lane) * a.g_rs + h] : 0.0f;
    const float bv = lane < L ? a.beta[(tb + lane) * a.beta_rs + h] : 0.0f;
    Gd[lane] = wave_prefix64((double)gv, lane);
    bt[lane] = bv;
  }
  __syncthreads();
  {  // row norms: 4 lanes per row, 32 elements each
    const int row = tid >> 2, qq = tid & 3;
    float sq = 0.0f, sk = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 xq = *reinterpret_cast<const uint4*>(Qs + row * LDQ + 32 * qq + 8 * u);
      const uint4 xk = *reinterpret_cast<const uint4*>(Ks + row * LDQ + 32 * qq + 8 * u);
      const uint32_t wq[4] = {xq.x, xq.y, xq.z, xq.w}, wk[4] = {xk.x, xk.y, xk.z, xk.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float q0 = M::dec(wq[e] & 0xffffu), q1 = M::dec(wq[e] >> 16);
        const float k0 = M::dec(wk[e] & 0xffffu), k1 = M::dec(wk[e] >> 16);
        sq += q0 * q0 + q1 * q1;
        sk += k0 * k0 + k1 * k1;
      }
    }
    sq += xor_lane<1>(sq);
    sq += xor_lane<2>(sq);
    sk += xor_lane<1>(sk);
    sk += xor_lane<2>(sk);
    if (qq == 0) {
      nq[row] = a.l2norm ? 1.0f / sqrtf(sq + a.l2_eps) : 1.0f;
      nk[row] = a.l2norm ? 1.0f / sqrtf(sk + a.l2_eps) : 1.0f;
    }
  }
  __syncthreads();
  if (w == 0) {  // per-token factors
    float* F = reinterpret_cast<float*>(rec + REC_F);
    const double gl = Gd[L - 1];
    const float eg = expf((float)Gd[lane]);
    F[lane] = eg * nk[lane];
    F[CK + lane] = eg * a.scale * nq[lane];
    F[2 * CK + lane] = expf((float)(gl - Gd[lane])) * nk[lane];
    F[3 * CK + lane] = lane == 0 ? expf((float)gl) : 0.0f;
  }

  // 20 tile products: K K^T (jobs 0..9) and Q K^T (jobs 10..19), lower tiles
  uint16_t* P = reinterpret_cast<uint16_t*>(rec + REC_P);
  for (int job = w; job < 20; job += 4) {
    const bool is_p = job >= 10;
    const int t = is_p ? job - 10 : job;
    const int ti = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
    const int tj = t - (ti * (ti + 1)) / 2;
    const uint16_t* X = is_p ? Qs : Ks;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      acc = M::mma(frag<TIN>(X, LDQ, 16 * ti, 32 * kk, lane),
                   frag<TIN>(Ks, LDQ, 16 * tj, 32 * kk, lane), acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * (lane >> 4) + r;
      const int j = 16 * tj + (lane & 15);
      const float e = expf((float)(Gd[i] - Gd[j]));
      if (is_p) {
        const float pv = j <= i ? acc[r] * a.scale * nq[i] * nk[j] * e : 0.0f;
        P[i * CK + j] = M::enc(pv);
      } else {
        Am[i * LDF + j] = j < i ? bt[i] * e * nk[i] * nk[j] * acc[r] : 0.0f;
      }
    }
  }
  // zero the strictly-upper 16x16 blocks of T and of P
  for (int idx = tid; idx < 6 * 256; idx += 256) {
    const int blk = idx >> 8, e = idx & 255;
    const int bi = blk < 3 ? 0 : blk < 5 ? 1 : 2;
    const int bj = blk < 3 ? blk + 1 : blk < 5 ? blk - 1 : 3;
    const int i = 16 * bi + (e >> 4), j = 16 * bj + (e & 15);
    Tm[i * LDF + j] = 0.0f;
    P[i * CK + j] = 0;
  }
  __syncthreads();

  // diagonal blocks of T = (I + A)^{-1}: forward substitution, one column per lane
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

  // off-diagonal blocks by distance d: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj,
  // 16x16x16 products on the f32 MFMA (A: lane (m = l%16, k = l/16),
  // B: lane (k = l/16, n = l%16), D: lane (m = 4 (l/16) + r, n = l%16))
  for (int d = 1; d < 4; ++d) {
    const int j = w, i = w + d;
    const bool active = i < 4;
    f32x4 r4 = {0.f, 0.f, 0.f, 0.f};
    if (active) {
      for (int k = j; k < i; ++k)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          r4 = __builtin_amdgcn_mfma_f32_16x16x4f32(
              Am[(16 * i + (lane & 15)) * LDF + 16 * k + 4 * s4 + (lane >> 4)],
              Tm[(16 * k + 4 * s4 + (lane >> 4)) * LDF + 16 * j + (lane & 15)], r4, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) Rs[w][(4 * (lane >> 4) + r) * 17 + (lane & 15)] = r4[r];
    }
    __syncthreads();
    if (active) {
      f32x4 t4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        t4 = __builtin_amdgcn_mfma_f32_16x16x4f32(
            Tm[(16 * i + (lane & 15)) * LDF + 16 * i + 4 * s4 + (lane >> 4)],
            Rs[w][(4 * s4 + (lane >> 4)) * 17 + (lane & 15)], t4, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Tm[(16 * i + 4 * (lane >> 4) + r) * LDF + 16 * j + (lane & 15)] = -t4[r];
    }
    __syncthreads();
  }

  // T_b = T diag(beta), split into high and low 16-bit parts
  uint16_t* Th = reinterpret_cast<uint16_t*>(rec + REC_TH);
  uint16_t* Tl = reinterpret_cast<uint16_t*>(rec + REC_TL);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = tid + 256 * u;
    const int i = idx >> 4, j4 = 4 * (idx & 15);
    const float4 t = *reinterpret_cast<const float4*>(Tm + i * LDF + j4);
    const float x[4] = {t.x * bt[j4], t.y * bt[j4 + 1], t.z * bt[j4 + 2], t.w * bt[j4 + 3]};
    uint16_t hh[4], ll[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hh[e] = M::enc(x[e]);
      ll[e] = M::enc(x[e] - M::dec(hh[e]));
    }
    *reinterpret_cast<uint2*>(Th + i * CK + j4) =
        make_uint2(hh[0] | ((uint32_t)hh[1] << 16), hh[2] | ((uint32_t)hh[3] << 16));
    *reinterpret_cast<uint2*>(Tl + i * CK + j4) =
        make_uint2(ll[0] | ((uint32_t)ll[1] << 16), ll[2] | ((uint32_t)ll[3] << 16));
  }
}

// ---------------------------------------------------------------------------
// the state walk
// ---------------------------------------------------------------------------
// K^T is stored [dk][token] with the 8-token groups XOR-swizzled by dk, so the
// transposed 2-byte writes of the four lane groups land in different banks and
// an 8-token operand read stays one contiguous 16-byte access.
__device__ __forceinline__ int kt_col(int dk, int token) { return token ^ (((dk >> 3) & 3) << 3); }

template <int NT>
struct WalkLds {
  static constexpr int BV = 16 * NT;            // state rows of the workgroup
  uint16_t Kt[DKC * LDT];                       // K^T of the chunk
  uint16_t Sh[2][BV * LDQ], Sl[2][BV * LDQ];    // S tile [dv][dk], double-buffered
  uint16_t Zh[BV * LDT], Zl[BV * LDT];          // Z^T  [dv][token]
  uint16_t Uh[BV * LDT], Ul[BV * LDT];          // U^T
  uint16_t Wh[BV * LDT], Wl[BV * LDT];          // (diag(fw) U)^T
};

// The chunk inputs a wave needs for its 16-row block: rows rb + lane % 16 for
// the A operands, rows rb + 4 (lane/16) + r for the elementwise work.
template <int NT>
struct ChunkRegs {
  uint4 q[4], k[4];    // Q, K rows, columns 32 kk + 8 (lane/16) .. +8
  uint4 th[2], tl[2];  // T_b rows, columns 32 kt + 8 (lane/16) .. +8
  uint4 p[2];          // P rows
  uint32_t v[NT][4];   // V[rb + 4 (lane/16) + r][dv0 + 16 nt + lane % 16]
  float4 fz, fo, fw;   // factors of rows rb + 4 (lane/16) .. +3
  float gc;
};

struct WalkCtx {
  const PrefillArgs* a;
  const char* recs;
  int64_t t_begin, t_end;
  int c0, h, hk, dv0, rb, nkt, lane;
};

__device__ __forceinline__ int chunk_len(const WalkCtx& c, int ch) {
  return (int)min((int64_t)CK, c.t_end - (c.t_begin + (int64_t)ch * CK));
}

__device__ __forceinline__ const char* chunk_rec(const WalkCtx& c, int ch) {
  return c.recs + ((int64_t)(c.c0 + ch) * c.a->hv + c.h) * REC_BYTES;
}

template <int NT>
__device__ __forceinline__ void fetch_qk(ChunkRegs<NT>& R, const WalkCtx& c, int ch) {
  const PrefillArgs& a = *c.a;
  const int64_t tb = c.t_begin + (int64_t)ch * CK;
  const int arow = min(c.rb + (c.lane & 15), chunk_len(c, ch) - 1);  // zeroed at use if >= L
  const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (tb + arow) * a.q_rs +
                       (int64_t)c.hk * DKC + 8 * (c.lane >> 4);
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + (tb + arow) * a.k_rs +
                       (int64_t)c.hk * DKC + 8 * (c.lane >> 4);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    R.q[kk] = *reinterpret_cast<const uint4*>(qp + 32 * kk);
    R.k[kk] = *reinterpret_cast<const uint4*>(kp + 32 * kk);
  }
}

__device__ __forceinline__ int rec_toff(const WalkCtx& c, int kt) {
  return 2 * ((c.rb + (c.lane & 15)) * CK + 8 * (c.lane >> 4) + 32 * kt);
}

// both k-steps are always loaded (for the first 32 rows the second one is the
// zero upper block), so every path issues the same memory operations
template <int NT>
__device__ __forceinline__ void fetch_t(ChunkRegs<NT>& R, const WalkCtx& c, int ch) {
  const char* rec = chunk_rec(c, ch);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    R.th[kt] = *reinterpret_cast<const uint4*>(rec + REC_TH + rec_toff(c, kt));
    R.tl[kt] = *reinterpret_cast<const uint4*>(rec + REC_TL + rec_toff(c, kt));
  }
}

template <int NT>
__device__ __forceinline__ void fetch_p(ChunkRegs<NT>& R, const WalkCtx& c, int ch) {
  const char* rec = chunk_rec(c, ch);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
    R.p[kt] = *reinterpret_cast<const uint4*>(rec + REC_P + rec_toff(c, kt));
}

template <int NT>
__device__ __forceinline__ void fetch_vf(ChunkRegs<NT>& R, const WalkCtx& c, int ch) {
  const PrefillArgs& a = *c.a;
  const int64_t tb = c.t_begin + (int64_t)ch * CK;
  const int L = chunk_len(c, ch);
  const uint16_t* vp = static_cast<const uint16_t*>(a.v) + (int64_t)c.h * a.dv + c.dv0 +
                       (c.lane & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int vrow = min(c.rb + 4 * (c.lane >> 4) + r, L - 1);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) R.v[nt][r] = vp[(tb + vrow) * a.v_rs + 16 * nt];
  }
  const float* F = reinterpret_cast<const float*>(chunk_rec(c, ch) + REC_F);
  const int frow = c.rb + 4 * (c.lane >> 4);
  R.fz = *reinterpret_cast<const float4*>(F + frow);
  R.fo = *reinterpret_cast<const float4*>(F + CK + frow);
  R.fw = *reinterpret_cast<const float4*>(F + 2 * CK + frow);
  R.gc = F[3 * CK];
}

__device__ __forceinline__ float f4(const float4& v, int r) {
  return r == 0 ? v.x : r == 1 ? v.y : r == 2 ? v.z : v.w;
}

// four consecutive 16-bit elements (rows i0..i0+3 of a transposed tile) as
// one 8-byte LDS store
__device__ __forceinline__ void store4(uint16_t* p, const uint16_t (&e)[4]) {
  *reinterpret_cast<uint2*>(p) =
      make_uint2((uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16));
}

// Output element type of the state walk.
template <int TOUT>
struct OutT {
  typedef uint16_t type;
  static __device__ __forceinline__ uint16_t cvt(float x) {
    return TOUT == kBF16 ? f32_to_bf16(x) : f32_to_f16(x);
  }
};
template <>
struct OutT<kF32> {
  typedef float type;
  static __device__ __forceinline__ float cvt(float x) { return x; }
};

// One workgroup walks one (sequence, v-head, 16 NT-row tile of S); wave w
// owns rows [16w, 16w + 16) of the chunk for X, Z, U and O, and the S tiles
// (mt, 2w + q) for mt < NT, q < 2.
// `dump` holds one 64 x 16 NT tile per workgroup: outputs of rows past the end
// of a sequence are written there instead of being skipped, so every chunk
// step issues the same number of stores and the compiler's memory-counter
// waits for the prefetched next chunk stay exact (a data-dependent store
// count makes it wait for all outstanding loads).
template <int TIN, int TOUT, int NT>
__global__ __launch_bounds__(256, 2) void chunk_state_kernel(PrefillArgs a, const int32_t* cs,
                                                             const int32_t* order,
                                                             const char* recs, int ntiles,
                                                             int max_chunks, float* dump) {
  constexpr int BV = 16 * NT;
  __shared__ __align__(16) WalkLds<NT> sm;
  using M = MT<TIN>;
  using x8 = typename M::x8;

  // XCD-aware mapping.  Workgroups are dealt round-robin to the 8 XCDs, each
  // with its own L2; the tiles of one v-head re-read the same per-chunk
  // records, and the v-heads of one GQA group the same q/k rows, so a unit
  // (sequence, q/k head) keeps all ratio * ntiles of its workgroups on one
  // XCD: block b -> xcd = b % 8, unit = (b / 8) / per_unit * 8 + xcd.
  const int ratio = a.hv / a.hk;
  const int per_unit = ratio * ntiles;
  const int xcd = blockIdx.x % kXcds;
  const int rblk = blockIdx.x / kXcds;
  const int unit = (rblk / per_unit) * kXcds + xcd;
  if (unit >= a.num_seqs * a.hk) return;
  const int j = rblk % per_unit;
  const int tile = j % ntiles;
  const int h = (unit % a.hk) * ratio + j / ntiles;
  const int s_rank = unit / a.hk;
  const int s = order[s_rank];
  const int sh = s_rank * a.hv + h;  // workgroup slot used for the dump area
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  WalkCtx c;
  c.a = &a;
  c.recs = recs;
  chunk_bounds(a, s, c.t_begin, c.t_end);
  c.c0 = cs[s];
  c.h = h;
  c.hk = h / ratio;
  c.dv0 = tile * BV;
  c.rb = 16 * w;
  c.nkt = (c.rb + 15) / 32 + 1;  // k-steps over tokens j <= i
  c.lane = lane;
  // a well-formed cu_seqlens gives c0 + nch <= max_chunks; a malformed one
  // (overlapping ranges) must still never index past the workspace
  const int nch =
      max(0, min((int)((c.t_end - c.t_begin + CK - 1) / CK), max_chunks - c.c0));
  const int64_t slot = a.idx ? (int64_t)a.idx[s] : (int64_t)s;
  const int64_t out_rs = (int64_t)a.hv * a.dv;

  if (slot < 0 || slot >= a.num_slots) {
    // caller error: NaN outputs for this tile, no state access
    for (int64_t t = c.t_begin + tid / BV; t < c.t_end; t += 256 / BV)
      store1(a.out, a.out_dt, t * out_rs + (int64_t)h * a.dv + c.dv0 + tid % BV,
             __builtin_nanf(""));
    return;
  }
  const bool init = a.has_init ? a.has_init[s] != 0 : true;
  float* Sg = a.pool + ((slot * a.hv + h) * a.dv + c.dv0) * DKC;
  const int rb = c.rb;
  const int nkt = c.nkt;
  using Ot = typename OutT<TOUT>::type;
  Ot* out = static_cast<Ot*>(a.out) + (int64_t)h * a.dv + c.dv0;
  Ot* dump_tile = reinterpret_cast<Ot*>(dump + ((int64_t)sh * ntiles + tile) * (CK * BV));

  // S tile (BV x 128) in MFMA accumulators: wave w holds tiles q = 2 mt + e
  // at (row block mt, column block 2w + e); element r of tile q is
  // S[16 mt + 4 (lane/16) + r][16 (2w + e) + lane % 16].
  f32x4 accs[2 * NT];
#pragma unroll
  for (int q = 0; q < 2 * NT; ++q) {
    const int mt = q >> 1, nt = 2 * w + (q & 1);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      accs[q][r] = init ? Sg[(16 * mt + 4 * (lane >> 4) + r) * DKC + 16 * nt + (lane & 15)] : 0.0f;
  }
  auto write_s_lds = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 2 * NT; ++q) {
      const int mt = q >> 1, nt = 2 * w + (q & 1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int off = (16 * mt + 4 * (lane >> 4) + r) * LDQ + 16 * nt + (lane & 15);
        const uint16_t hb = M::enc(accs[q][r]);
        sm.Sh[buf][off] = hb;
        sm.Sl[buf][off] = M::enc(accs[q][r] - M::dec(hb));
      }
    }
  };
  // Q, K, V and the factors are fetched one chunk ahead; T_b and P (needed
  // only from the second phase on) at the start of their own chunk.
  auto fetch_ahead = [&](ChunkRegs<NT>& R, int ch) {
    fetch_qk(R, c, ch);
    fetch_vf(R, c, ch);
  };

  // One chunk with its inputs in `R`; the next chunk's Q, K, V and factors
  // are requested into `N` first.  The loop below alternates the two register
  // sets so that no loaded register is copied across iterations (a copy would
  // wait for the whole prefetch).
  auto step = [&](ChunkRegs<NT>& R, ChunkRegs<NT>& N, int ch) {
    const int cb = ch & 1;
    const int64_t tb = c.t_begin + (int64_t)ch * CK;
    const int L = chunk_len(c, ch);
    fetch_t(R, c, ch);
    fetch_p(R, c, ch);
    fetch_ahead(N, min(ch + 1, nch - 1));  // the last step re-fetches its own chunk
    // rows of this wave past the end of the sequence: zero operands
    if (rb + (lane & 15) >= L) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        R.q[kk] = make_uint4(0, 0, 0, 0);
        R.k[kk] = make_uint4(0, 0, 0, 0);
      }
    }

    // ---- X = K S^T and QS = Q S^T of the row block; K^T to LDS; Z ----
    f32x4 accq[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 accx = {0.f, 0.f, 0.f, 0.f};
      accq[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const x8 shi = frag<TIN>(sm.Sh[cb], LDQ, 16 * nt, 32 * kk, lane);
        const x8 slo = frag<TIN>(sm.Sl[cb], LDQ, 16 * nt, 32 * kk, lane);
        const x8 kf = __builtin_bit_cast(x8, R.k[kk]);
        const x8 qf = __builtin_bit_cast(x8, R.q[kk]);
        accx = M::mma(kf, shi, accx);
        accq[nt] = M::mma(qf, shi, accq[nt]);
        accx = M::mma(kf, slo, accx);
        accq[nt] = M::mma(qf, slo, accq[nt]);
      }
      uint16_t zh[4], zl[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = rb + 4 * (lane >> 4) + r;
        const float vv = i < L ? M::dec(R.v[nt][r]) : 0.0f;
        const float z = vv - f4(R.fz, r) * accx[r];
        zh[r] = M::enc(z);
        zl[r] = M::enc(z - M::dec(zh[r]));
      }
      const int off = (16 * nt + (lane & 15)) * LDT + rb + 4 * (lane >> 4);
      store4(sm.Zh + off, zh);
      store4(sm.Zl + off, zl);
    }
    {
      const int tok = rb + (lane & 15);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint32_t kw[4] = {R.k[kk].x, R.k[kk].y, R.k[kk].z, R.k[kk].w};
        const int d0 = 32 * kk + 8 * (lane >> 4);
        const int col = kt_col(d0, tok);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sm.Kt[(d0 + 2 * e) * LDT + col] = (uint16_t)(kw[e] & 0xffffu);
          sm.Kt[(d0 + 2 * e + 1) * LDT + col] = (uint16_t)(kw[e] >> 16);
        }
      }
    }
    lds_barrier();

    // ---- U = T_b Z (row block); U^T and (diag(fw) U)^T to LDS ----
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 accu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (kt < nkt) {
          const x8 th = __builtin_bit_cast(x8, R.th[kt]);
          const x8 tl = __builtin_bit_cast(x8, R.tl[kt]);
          const x8 zh = frag<TIN>(sm.Zh, LDT, 16 * nt, 32 * kt, lane);
          const x8 zl = frag<TIN>(sm.Zl, LDT, 16 * nt, 32 * kt, lane);
          accu = M::mma(th, zh, accu);
          accu = M::mma(th, zl, accu);
          accu = M::mma(tl, zh, accu);
        }
      }
      uint16_t uh[4], ul[4], wh[4], wl[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float u = accu[r];
        uh[r] = M::enc(u);
        ul[r] = M::enc(u - M::dec(uh[r]));
        const float up = u * f4(R.fw, r);
        wh[r] = M::enc(up);
        wl[r] = M::enc(up - M::dec(wh[r]));
      }
      const int off = (16 * nt + (lane & 15)) * LDT + rb + 4 * (lane >> 4);
      store4(sm.Uh + off, uh);
      store4(sm.Ul + off, ul);
      store4(sm.Wh + off, wh);
      store4(sm.Wl + off, wl);
    }
    lds_barrier();

    // ---- outputs of the row block; state update; S to the other buffer ----
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acco = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (kt < nkt) {
          const x8 pf = __builtin_bit_cast(x8, R.p[kt]);
          acco = M::mma(pf, frag<TIN>(sm.Uh, LDT, 16 * nt, 32 * kt, lane), acco);
          acco = M::mma(pf, frag<TIN>(sm.Ul, LDT, 16 * nt, 32 * kt, lane), acco);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = rb + 4 * (lane >> 4) + r;
        const float o = f4(R.fo, r) * accq[nt][r] + acco[r];
        Ot* dst = i < L ? out + (tb + i) * out_rs + 16 * nt + (lane & 15)
                        : dump_tile + i * BV + 16 * nt + (lane & 15);
        *dst = OutT<TOUT>::cvt(o);
      }
    }
#pragma unroll
    for (int q = 0; q < 2 * NT; ++q) {
      const int mt = q >> 1, nt = 2 * w + (q & 1);
      const int dk = 16 * nt + (lane & 15);
      f32x4 acc = accs[q];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] *= R.gc;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const x8 kf = *reinterpret_cast<const x8*>(
            sm.Kt + dk * LDT + kt_col(dk, 32 * kt + 8 * (lane >> 4)));
        acc = M::mma(frag<TIN>(sm.Wh, LDT, 16 * mt, 32 * kt, lane), kf, acc);
        acc = M::mma(frag<TIN>(sm.Wl, LDT, 16 * mt, 32 * kt, lane), kf, acc);
      }
      accs[q] = acc;
    }
    write_s_lds(cb ^ 1);
    lds_barrier();
  };

  write_s_lds(0);
  ChunkRegs<NT> RA, RB;
  if (nch > 0) fetch_ahead(RA, 0);
  __syncthreads();
  for (int ch = 0; ch < nch; ch += 2) {
    step(RA, RB, ch);
    if (ch + 1 < nch) step(RB, RA, ch + 1);
  }

  // final state
#pragma unroll
  for (int q = 0; q < 2 * NT; ++q) {
    const int mt = q >> 1, nt = 2 * w + (q & 1);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      Sg[(16 * mt + 4 * (lane >> 4) + r) * DKC + 16 * nt + (lane & 15)] = accs[q][r];
  }
}

int64_t max_chunks(int64_t total_tokens, int64_t num_seqs) {
  return (total_tokens + CK - 1) / CK + num_seqs;
}

size_t meta_bytes(int64_t num_seqs) { return (size_t)((2 * num_seqs + 1) * 4 + 255) / 256 * 256; }

size_t dump_bytes(int64_t num_seqs, int hv, int dv) {
  return (size_t)num_seqs * hv * (dv / BVT) * CK * BVT * sizeof(float);
}

template <int TIN>
hipError_t launch_chunked_t(const PrefillArgs& a, void* ws, hipStream_t stream) {
  int32_t* cs = static_cast<int32_t*>(ws);
  int32_t* order = cs + a.num_seqs + 1;
  char* recs = static_cast<char*>(ws) + meta_bytes(a.num_seqs);
  const int64_t mc = max_chunks(a.total_tokens, a.num_seqs);
  float* dump = reinterpret_cast<float*>(recs + (size_t)mc * a.hv * REC_BYTES);
  hipLaunchKernelGGL(chunk_meta_kernel, dim3(1), dim3(256), 0, stream, a, cs, order);
  hipLaunchKernelGGL((chunk_prep_kernel<TIN>), dim3((unsigned)mc, (unsigned)a.hv), dim3(256), 0,
                     stream, a, (const int32_t*)cs, recs);
  const int ntiles = a.dv / BVT;
  const int64_t units = a.num_seqs * a.hk;
  const int64_t blocks = (units + kXcds - 1) / kXcds * kXcds * (a.hv / a.hk) * ntiles;
  if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (a.out_dt == kF32)
    hipLaunchKernelGGL((chunk_state_kernel<TIN, kF32, WALK_NT>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a, (const int32_t*)cs, (const int32_t*)order, (const char*)recs,
                       ntiles, (int)mc, dump);
  else
    hipLaunchKernelGGL((chunk_state_kernel<TIN, TIN, WALK_NT>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a, (const int32_t*)cs, (const int32_t*)order, (const char*)recs,
                       ntiles, (int)mc, dump);
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
  return meta_bytes(num_seqs) + (size_t)max_chunks(total_tokens, num_seqs) * (size_t)hv * REC_BYTES +
         dump_bytes(num_seqs, hv, dv);
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
