// gdn_chunked.hip -- chunk-parallel varlen prefill with the dense products on
// MFMA (v_mfma_f32_16x16x32_{bf16,f16}), for Dk = 128, Dv a multiple of 16 and
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
//                       the device (no host synchronisation), and the order
//                       of the sequences by length;
//   chunk_prep_kernel   one workgroup per (chunk, q/k head): K K^T and Q K^T on
//                       MFMA once per GQA group, then per v-head the strictly
//                       lower A, T = (I + A)^{-1} by blocked forward
//                       substitution (16x16 blocks), T_b = T diag(beta), P and
//                       the per-token factors to a record in the workspace --
//                       all of it independent of the state;
//   chunk_state_kernel  one workgroup per (sequence, v-head, block of 16 NW
//                       state rows) walks the chunks in order; each wave keeps
//                       its 16 rows of S for all keys in MFMA accumulators:
//                         X = K S^T,  Z = V - diag(e^G n_k) X,  U = T_b Z,
//                         O = diag(e^G scale n_q) Q S^T + P U,
//                         S = e^{G_C} S + (diag(e^{G_C - G} n_k) U)^T K.
//                       Forming U as T_b (V - ...) never builds the 64 x 128
//                       matrix T diag(beta e^G) K, so each wave does only work
//                       proportional to its own 16 rows.
// Precision: the raw 16-bit q/k/v are exact MFMA operands; the L2 norms enter
// as diagonal scalings; an f32 operand (S, T_b, Z, U) is split into a 16-bit
// high part and a 16-bit remainder, and the products keep hi*hi + hi*lo +
// lo*hi (both sides computed) or hi + lo (one side raw), which carries about
// 16 significant bits -- the state is accumulated in f32 throughout.  The
// cumulative gate G is summed in f64 so differences G_i - G_j stay exact even
// when a head's gate is thousands per chunk.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_prefill_gate.h"

namespace gdn {
namespace {

constexpr int CK = 64;        // tokens per chunk
constexpr int DKC = 128;      // key head size served here
#ifndef GDN_WALK_NW
#define GDN_WALK_NW 4
#endif
#ifndef GDN_WALK_NB
#define GDN_WALK_NB 1
#endif
#ifndef GDN_WALK_MINB
#define GDN_WALK_MINB 1
#endif
constexpr int WALK_NW = GDN_WALK_NW;      // compute waves per state-walk workgroup (plus one load wave)
constexpr int WALK_NB = GDN_WALK_NB;      // 16-row state blocks per wave
constexpr int WALK_MINB = GDN_WALK_MINB;  // register budget: as for this many workgroups per CU
constexpr int WALK_BV = 16 * WALK_NW * WALK_NB;  // state rows per workgroup
constexpr int kXcds = 8;      // accelerator complex dies (separate L2s) on MI355X

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// Workgroup barrier ordering LDS only.  __syncthreads() also waits for every
// outstanding global access (the output stores, say); all communication
// between the waves here goes through LDS, so global accesses may stay in
// flight, and a wave whose loads must have landed waits for them itself.
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
// Per-call metadata in the workspace, formed on the device from cu_seqlens
// (no host synchronisation):
//   cs[s]    number of chunks of sequences before s; cs[n] = total;
//   order[r] the sequence with the r-th most chunks (ties by index) when
//            n <= kOrderMax, else r;
//   ocs[r]   number of chunks of the sequences ranked before r;
//   info[0]  split rank k: ranks [0, k) (the longest sequences) are walked as
//            soon as their own records exist, while the records and walks of
//            the other ranks proceed beside them on the remaining CUs;
//   info[1]  ks: ranks [0, ks) are split into info[2] = S segments each, of
//            info[3 + r] chunks (the last one may be shorter);
// The walk starts the longest sequences first, since the longest one bounds
// the whole prefill.
//
// Segments.  Over a run of tokens the state maps affinely, S_out = S_in M +
// S_loc, where M = prod_t decay_t (I - beta_t k_t k_t^T) (Dk x Dk) is the walk
// of the identity with v = 0 and S_loc the walk from zero.  A split sequence is
// walked in two phases: A) the state alone (no outputs) over segment 0 from
// the real initial state, giving S_in of segment 1, and for each middle
// segment j its S_loc and M, all at once; B) every segment j with its outputs,
// from its exact entry state S_in(1) M_1 ... + (folded in a prologue:
// S <- S M_i + S_loc,i for i = 1 .. j - 1).  The chain of chunk steps of a
// sequence of C chunks shrinks from C to about (3/4 + 1) C / S, for about
// (3/4 (2 S - 3) + S) C / S workgroup steps in all instead of C.
// ---------------------------------------------------------------------------
constexpr int kOrderMax = 1024;
constexpr int kSplitMax = 8;   // most ranks the early walk may take
constexpr int kSegRanks = 2;   // most ranks (the longest) a call splits into segments
constexpr int kSegMax = 5;     // most segments per split rank
constexpr int kInfoWords = 3 + kSegRanks;

// How far a call of these sizes may split: S segments need at least 2 S
// chunks, so at most (chunks + 1) / 2 segments and total_tokens / 256 + 1
// split ranks.  The workspace holds 2 (S - 1) f32 states per split rank and
// v-head: the initial state, the entry state of segment 1, and S_loc and M^T
// of each middle segment.
struct SegBounds {
  int ranks, smax;
  int slots() const { return ranks > 0 ? 2 * (smax - 1) : 0; }
};
inline SegBounds seg_bounds(int64_t total_tokens, int64_t num_seqs) {
  const int64_t chunks = (total_tokens + CK - 1) / CK;
  const int smax = (int)std::min<int64_t>(kSegMax, (chunks + 1) / 2);
  const int ranks = (int)std::min<int64_t>({(int64_t)kSegRanks, num_seqs, total_tokens / (4 * CK) + 1});
  if (smax < 2 || num_seqs > kOrderMax) return {0, 1};
  return {ranks, smax};
}

struct MetaPtrs {
  int32_t *cs, *order, *ocs, *info;
};

__host__ __device__ inline MetaPtrs meta_ptrs(void* ws, int64_t n) {
  int32_t* p = static_cast<int32_t*>(ws);
  return {p, p + n + 1, p + 2 * n + 1, p + 3 * n + 2};  // info: kInfoWords words
}

// A DPP move of an int32; lanes the move does not reach read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int32_t dpp_i32(int32_t x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, true);
}

// block-wide inclusive scan of one value per thread (256 threads): each
// wave scans its 64 values with DPP row shifts and row broadcasts, then adds
// the totals of the waves before it (one barrier; part[0..3] is free again
// when it returns)
__device__ __forceinline__ int32_t block_scan256(int32_t v, int32_t* part) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v += dpp_i32<0x111, 0xF>(v);  // row_shr:1
  v += dpp_i32<0x112, 0xF>(v);  // row_shr:2
  v += dpp_i32<0x114, 0xF>(v);  // row_shr:4
  v += dpp_i32<0x118, 0xF>(v);  // row_shr:8
  v += dpp_i32<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_i32<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  if (lane == 63) part[w] = v;
  __syncthreads();
  for (int i = 0; i < w; ++i) v += part[i];
  __syncthreads();
  return v;
}

// The schedule of a call, from a cost model in units of one chunk step of one
// walk workgroup (measured on MI355X: a walk step takes about 2.4 us, the
// prep of one (chunk, v-head) record on one CU about as long, a step that
// updates the state alone about 0.9 of a full one, and folding one middle
// segment's transition into a segment's entry state about one step).  W
// workgroups walk one sequence (or segment, or one middle segment's M);
// workgroups of a phase beyond the CUs it has wait for a second round.
// Chooses
//   k   the split rank (0: everything in one order; the host passes kmax = 0
//       when it will not use a second stream),
//   ks  the longest ranks split into S segments each (ks <= k when k > 0, so
//       a split sequence's two phases stay in one stream order).
// Ranks are sorted by length, so the longest unsplit rank is rank ks.
struct Plan {
  int k, ks, S;
};

constexpr double kStateStep = 0.9;  // a state-only walk step against a full one
constexpr double kFoldStep = 1.0;   // folding one transition into an entry state

// Walks of ranks [0, r1) on `cap` CUs, ranks [0, ks) split S ways.
__device__ double plan_walks(const int32_t* ocs, int r1, int ks, int S, double W, double cap) {
  double tA = 0.0, tB = 0.0, work = 0.0;
  if (ks > 0) {
    double Lmax = 0.0;
    for (int r = 0; r < ks; ++r) {
      const double L = ceil((double)(ocs[r + 1] - ocs[r]) / S);
      Lmax = fmax(Lmax, L);
      work += W * S * L;
    }
    tA = kStateStep * Lmax * ceil(W * ks * (2 * S - 3) / cap);
    tB = Lmax * ceil(W * ks * S / cap) + kFoldStep * (S - 2);
  }
  const double chain = ks < r1 ? (double)(ocs[ks + 1] - ocs[ks]) : 0.0;
  work += W * (double)(ocs[r1] - ocs[ks]);
  return tA + fmax(fmax(tB, chain), work / cap);
}

// The cost of candidate `c` (k, ks, S), or a huge value when it is not allowed.
// Candidates: c = (k * 3 + ks) * kSegMax + (S - 1) for k in [0, kSplitMax + 1]
// (k = kSplitMax + 1 stands for k = n: every rank early).
constexpr int kPlanCands = (kSplitMax + 2) * 3 * kSegMax;
static_assert(kPlanCands <= 256 && kSegRanks <= 2, "one plan candidate per metadata thread");
__device__ double plan_cost(int c, const int32_t* ocs, int n, int hv, double W, double NC,
                            int kmax, int ksmax, int smax, Plan& p) {
  const double no = 1e300;
  int k = c / (3 * kSegMax);
  const int ks = (c / kSegMax) % 3, S = c % kSegMax + 1;
  if ((ks == 0) != (S == 1) || S > smax || ks > ksmax || ks > n) return no;
  for (int r = 0; r < ks; ++r)
    if (ocs[r + 1] - ocs[r] < 2 * S) return no;
  const double C = ocs[n], H = hv;
  const double records = C * H / NC;
  if (k == kSplitMax + 1) {  // every rank early: one stream order, with a second stream at hand
    if (kmax == 0 || n > kSplitMax || ks == 0) return no;
    p = {n, ks, S};
    return records + plan_walks(ocs, n, ks, S, W, NC) + 2.0;  // the empty second part
  }
  if (k == 0) {
    if (kmax > 0 && ks > 0) return no;  // the second stream's order cannot split
    p = {0, ks, S};
    return records + plan_walks(ocs, n, ks, S, W, NC);
  }
  if (k > kmax || k >= n || ks > k) return no;
  const double wgs = fmax(W * ks * (2 * S - 3), W * (ks * S + (k - ks)));
  if (wgs > NC / 2) return no;
  const double F = NC - wgs, CL = ocs[k];
  const double head = CL * H / NC;
  const double t1 = head + plan_walks(ocs, k, ks, S, W, NC / 2);
  const double t2 = head + (C - CL) * H / F + fmax((double)(ocs[k + 1] - ocs[k]), (C - CL) * W / F);
  p = {k, ks, S};
  return fmax(t1, t2) + 4.0;  // the second stream's launches and joins
}

// The metadata kernel's LDS, also carved out of the prep kernel's when the
// prep forms the metadata itself (one stream order).
struct MetaLds {
  int32_t part[256];
  // Up to kOrderMax sequences the three tables are built in LDS and copied
  // out once at the end (no global round trips between the steps).
  int32_t l_cs[kOrderMax + 1], l_order[kOrderMax], l_ocs[kOrderMax + 1];
  Plan plans[256];
  double wcost[4];
  int widx[4];
};

// Chunk offsets per sequence, the order of the sequences by length, the chunk
// offsets in that order and the plan, by one workgroup of 256 threads.
__device__ __forceinline__ void meta_body(const PrefillArgs& a, const MetaPtrs& m, int ntiles,
                                          int ncu, int kmax, int ksmax, int smax, MetaLds& L) {
  const int n = (int)a.num_seqs;
  const bool small = n <= kOrderMax;
  int32_t* const cs = small ? L.l_cs : m.cs;
  int32_t* const order = small ? L.l_order : m.order;
  int32_t* const ocs = small ? L.l_ocs : m.ocs;
  int32_t carry = 0;
  if (threadIdx.x == 0) cs[0] = 0;
  for (int base = 0; base < n; base += 256) {
    const int s = base + (int)threadIdx.x;
    int32_t c = 0;
    if (s < n) {
      int64_t t0, t1;
      chunk_bounds(a, s, t0, t1);
      c = (int32_t)((t1 - t0 + CK - 1) / CK);
    }
    const int32_t incl = block_scan256(c, L.part);
    if (s < n) cs[s + 1] = carry + incl;
    if (threadIdx.x == 255) L.part[0] = incl;
    __syncthreads();
    carry += L.part[0];
    __syncthreads();
  }
  __syncthreads();
  for (int s = threadIdx.x; s < n; s += 256) {
    int rank = s;
    if (small) {
      const int cnt = cs[s + 1] - cs[s];
      rank = 0;
      for (int t = 0; t < n; ++t) {
        const int ct = cs[t + 1] - cs[t];
        rank += (ct > cnt) || (ct == cnt && t < s);
      }
    }
    order[rank] = s;
  }
  __syncthreads();
  // chunk offsets in rank order
  carry = 0;
  if (threadIdx.x == 0) ocs[0] = 0;
  for (int base = 0; base < n; base += 256) {
    const int r = base + (int)threadIdx.x;
    int32_t c = 0;
    if (r < n) {
      const int s = order[r];
      c = cs[s + 1] - cs[s];
    }
    const int32_t incl = block_scan256(c, L.part);
    if (r < n) ocs[r + 1] = carry + incl;
    if (threadIdx.x == 255) L.part[0] = incl;
    __syncthreads();
    carry += L.part[0];
    __syncthreads();
  }
  __syncthreads();
  // the plan: one candidate per thread, then the cheapest (ties: the lowest
  // index), by shuffles within each wave and then over the four waves
  {
    Plan p = {0, 0, 1};
    double t = 1e300;
    if (small && threadIdx.x < kPlanCands)
      t = plan_cost(threadIdx.x, ocs, n, a.hv, (double)a.hv * ntiles, ncu, kmax, ksmax, smax, p);
    L.plans[threadIdx.x] = p;
    int bi = threadIdx.x;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const double to = __shfl_xor(t, off, 64);
      const int io = __shfl_xor(bi, off, 64);
      if (to < t || (to == t && io < bi)) {
        t = to;
        bi = io;
      }
    }
    if ((threadIdx.x & 63) == 0) {
      L.wcost[threadIdx.x >> 6] = t;
      L.widx[threadIdx.x >> 6] = bi;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = L.wcost[0];
    int bi = L.widx[0];
    for (int i = 1; i < 4; ++i)
      if (L.wcost[i] < t) {
        t = L.wcost[i];
        bi = L.widx[i];
      }
    const Plan p = t < 1e299 ? L.plans[bi] : Plan{0, 0, 1};
    m.info[0] = p.k;
    m.info[1] = p.ks;
    m.info[2] = p.S;
    for (int r = 0; r < kSegRanks; ++r)
      m.info[3 + r] = r < p.ks ? (ocs[r + 1] - ocs[r] + p.S - 1) / p.S : 0;
  }
  if (small) {
    for (int i = threadIdx.x; i <= n; i += 256) {
      m.cs[i] = L.l_cs[i];
      m.ocs[i] = L.l_ocs[i];
      if (i < n) m.order[i] = L.l_order[i];
    }
  }
}

__global__ __launch_bounds__(256) void chunk_meta_kernel(PrefillArgs a, MetaPtrs m, int ntiles,
                                                         int ncu, int kmax, int ksmax,
                                                         int smax) {
  __shared__ MetaLds L;
  meta_body(a, m, ntiles, ncu, kmax, ksmax, smax, L);
}

// The range of rank-order chunks [c0, c1) of a launch part: 0 = the ranks
// walked early, 1 = the others, 2 = all.
__device__ __forceinline__ void part_chunks(const MetaPtrs& m, int n, int part, int& c0, int& c1) {
  const int k = part == 2 ? 0 : m.info[0];
  c0 = part == 1 ? m.ocs[k] : 0;
  c1 = part == 0 ? m.ocs[k] : m.ocs[n];
}

// A DPP move of an f64 (both halves); lanes the move does not reach read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xF,
                                             true);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// inclusive prefix sum of 64 values held one per lane of a wave, in f64:
// shifts by 1, 2, 4, 8 within each row of 16 lanes, then the last lane of
// row 0 (row 2) added to row 1 (row 3), then lane 31 added to rows 2 and 3
__device__ __forceinline__ double wave_prefix64(double x) {
  x += dpp_f64<0x111, 0xF>(x);  // row_shr:1
  x += dpp_f64<0x112, 0xF>(x);  // row_shr:2
  x += dpp_f64<0x114, 0xF>(x);  // row_shr:4
  x += dpp_f64<0x118, 0xF>(x);  // row_shr:8
  x += dpp_f64<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_f64<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
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
// Each [64][64] part is stored as its 4 x 4 grid of 16 x 16 blocks, 512 bytes
// each (rows of 32 bytes inside), so every block that is written or read is
// four whole 128-byte lines.  T_b and P are lower triangular: their blocks
// (0, 1) and (2, 3), above the diagonal inside the diagonal 32 x 32
// quadrants, are zero and neither written nor read (the walk's loads of them
// fall outside the record's buffer range and arrive as zeros).  The walk
// multiplies T_b and P only in 32-token block pairs on or below the
// diagonal, so their upper-right 32 x 32 quadrants (blocks (0, 2), (0, 3),
// (1, 2), (1, 3)) are free.  A 16-bit output needs only P's high part; for an
// f32 output the low part of P (P - high, rounded to 16 bits) is kept there:
// its quadrant (0, 0) in T_b-high's free quadrant, (1, 0) in T_b-low's and
// (1, 1) in P's, element (i, j) at row i % 32, column 32 + j % 32.  For 16-bit
// outputs the free quadrants are never written or read.
// ---------------------------------------------------------------------------
constexpr int REC_TH = 0;
constexpr int REC_TL = CK * CK * 2;
constexpr int REC_P = 2 * CK * CK * 2;
constexpr int REC_F = 3 * CK * CK * 2;
constexpr int REC_BYTES = REC_F + 4 * CK * 4;

// 16-bit element index of (i, j) in a record part: block (i / 16, j / 16) of
// the part's 4 x 4 grid of 256-element blocks, row-major inside the block.
__device__ __forceinline__ int rec_elem(int i, int j) {
  return (((i >> 4) << 2) + (j >> 4)) * 256 + (i & 15) * 16 + (j & 15);
}

// One workgroup per (chunk, q/k head): the raw products K K^T and Q K^T of the
// chunk are shared by the v-heads of the GQA group, so they are formed once
// (each wave keeps the A and P tiles of the same blocks in registers, so one
// exponential serves both) and then, head by head, scaled by that head's
// gates and betas, solved and written out.  The gate prefix sums and per-token
// factors of up to four heads are formed at once, one head per wave.
//
// LDS: Q and K are needed only for the products; the lower 16x16 blocks of A
// and T and the per-wave partial products then reuse their space.  About
// 36 KB in all, so four workgroups share a CU.
constexpr double kLog2e = 1.4426950408889634;  // log2(e)
constexpr int LDB = 20;         // padded f32 row of a 16x16 block of A or T
constexpr int kPrepHeads = 4;   // v-heads whose factors are formed at once (one per wave)

struct PrepLds {
  union {
    struct {
      uint16_t Q[CK * DKC], K[CK * DKC];  // [token][key], 16-byte chunks XOR-swizzled by row
    } qk;
    struct {
      float A[10][16 * LDB];  // lower blocks (bi >= bj) at bi (bi + 1) / 2 + bj
      float T[10][16 * LDB];
      float R[4][16 * 17];    // each wave's partial sum of an off-diagonal block
    } at;
  } u;
  float nq[CK], nk[CK];
  double Gd[kPrepHeads][CK];  // gate prefix sums in base-2 units, G log2(e)
  float bt[kPrepHeads][CK];
};

// the 16-byte chunk of a Q/K row where logical chunk `chunk` is kept: a
// 16-row operand read (or a row's four quarter reads) then touches 16
// distinct 4-bank groups
__device__ __forceinline__ int qk_chunk(int row, int chunk) { return chunk ^ (row & 15); }

// MFMA operand (16 rows x 32 k) from swizzled Q or K: lane l takes row
// r0 + l % 16, elements k0 + 8 (l / 16) .. +8
template <int TIN>
__device__ __forceinline__ typename MT<TIN>::x8 frag_qk(const uint16_t* m, int r0, int k0, int lane) {
  const int row = r0 + (lane & 15);
  return *reinterpret_cast<const typename MT<TIN>::x8*>(
      m + row * DKC + 8 * qk_chunk(row, (k0 >> 3) + (lane >> 4)));
}

__device__ __forceinline__ int lower_blk(int bi, int bj) { return (bi * (bi + 1)) / 2 + bj; }

// One (chunk, q/k head) unit: chunk c (record index) of tokens [tb, tb + L).
template <int TIN>
__device__ __forceinline__ void prep_unit(const PrefillArgs& a, char* recs, PrepLds& sh, int c,
                                          int hk, int64_t tb, int L) {
  using M = MT<TIN>;
  const int ratio = a.hv / a.hk;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool plo = a.out_dt == kF32;
  uint16_t* Qs = sh.u.qk.Q;
  uint16_t* Ks = sh.u.qk.K;

  // gate and beta of this wave's head in the first group (one token per
  // lane), in flight while Q and K are staged
  float gv = 0.0f, bv = 0.0f;
  auto load_gb = [&](int q) {
    const int jh = kPrepHeads * q + w;
    gv = 0.0f;
    bv = 0.0f;
    if (jh < ratio && lane < L) token_gate(a, tb + lane, hk * ratio + jh, gv, bv);
  };
  load_gb(0);

  // stage Q and K, rows past the sequence zeroed (all loads issued before any is used)
  {
    u32x4 qv[4], kv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = tid + 256 * k;
      const int64_t t = tb + min(idx >> 4, L - 1);
      qv[k] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + t * a.q_rs +
                                              (int64_t)hk * DKC + 8 * (idx & 15));
      kv[k] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.k) + t * a.k_rs +
                                              (int64_t)hk * DKC + 8 * (idx & 15));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = tid + 256 * k;
      const int row = idx >> 4, p = qk_chunk(row, idx & 15);
      const u32x4 zero = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(Qs + row * DKC + 8 * p) = row < L ? qv[k] : zero;
      *reinterpret_cast<u32x4*>(Ks + row * DKC + 8 * p) = row < L ? kv[k] : zero;
    }
  }
  __syncthreads();
  {  // row norms: 4 lanes per row, 32 elements each
    const int row = tid >> 2, qq = tid & 3;
    float sq = 0.0f, sk = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = qk_chunk(row, 4 * qq + k);
      const uint4 xq = *reinterpret_cast<const uint4*>(Qs + row * DKC + 8 * p);
      const uint4 xk = *reinterpret_cast<const uint4*>(Ks + row * DKC + 8 * p);
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
      sh.nq[row] = a.l2norm ? 1.0f / sqrtf(sq + a.l2_eps) : 1.0f;
      sh.nk[row] = a.l2norm ? 1.0f / sqrtf(sk + a.l2_eps) : 1.0f;
    }
  }

  // the lower 16x16 blocks t = 0..9 of K K^T and Q K^T: wave w owns blocks
  // w, w + 4, w + 8 (< 10), each formed transposed (the products taken as
  // K_j . K_i and K_j . Q_i) so that a lane holds one row i = 16 ti + l % 16
  // and four consecutive columns j = 16 tj + 4 (l/16) + r: the row's four
  // values then leave in one store
  f32x4 accA[3], accP[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int t = w + 4 * k;
    accA[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
    accP[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (t < 10) {
      const int ti = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
      const int tj = t - (ti * (ti + 1)) / 2;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const typename M::x8 kj = frag_qk<TIN>(Ks, 16 * tj, 32 * kk, lane);
        accA[k] = M::mma(kj, frag_qk<TIN>(Ks, 16 * ti, 32 * kk, lane), accA[k]);
        accP[k] = M::mma(kj, frag_qk<TIN>(Qs, 16 * ti, 32 * kk, lane), accP[k]);
      }
    }
  }
  __syncthreads();  // Q and K are dead from here on; the norms are visible

  // prefix sums of the gates and the per-token factors of heads
  // kPrepHeads q .. +3, wave w forming head kPrepHeads q + w
  auto factors = [&](int q) {
    const int jh = kPrepHeads * q + w;
    if (jh < ratio) {
      const int h = hk * ratio + jh;
      char* rec = recs + ((int64_t)c * a.hv + h) * REC_BYTES;
      const double gcum = wave_prefix64((double)gv);
      sh.Gd[w][lane] = gcum * kLog2e;
      sh.bt[w][lane] = bv;
      const double gl = __shfl(gcum, L - 1, 64);
      const float eg = expf((float)gcum);
      float* F = reinterpret_cast<float*>(rec + REC_F);
      F[lane] = eg * sh.nk[lane];
      F[CK + lane] = eg * a.scale * sh.nq[lane];
      F[2 * CK + lane] = expf((float)(gl - gcum)) * sh.nk[lane];
      F[3 * CK + lane] = lane == 0 ? expf((float)gl) : 0.0f;
    }
    load_gb(q + 1);  // the next group's, a group ahead
  };
  factors(0);
  __syncthreads();

  float* const Ab = &sh.u.at.A[0][0];
  float* const Tb = &sh.u.at.T[0][0];
  constexpr int BLK = 16 * LDB;
  for (int jh = 0; jh < ratio; ++jh) {
    const int hs = jh % kPrepHeads;
    if (jh > 0 && hs == 0) {
      factors(jh / kPrepHeads);
      __syncthreads();
    }
    // lane-derived indices are formed afresh for each head: hoisted out of
    // the loop they would hold more registers than four workgroups per CU allow
    int tid_h = tid;
    asm volatile("" : "+v"(tid_h));
    const int lane = tid_h & 63;
    const int g = lane >> 4, cl = lane & 15;
    const int h = hk * ratio + jh;
    char* rec = recs + ((int64_t)c * a.hv + h) * REC_BYTES;
    uint16_t* Pg = reinterpret_cast<uint16_t*>(rec + REC_P);
    // an f32 output also keeps P's low part, in the free quadrants (quadrant
    // (qi, qj) in the free quadrant of record part qi + qj)
    auto plo_dst = [&](int i, int j) {
      const int part = (i >> 5) + (j >> 5);
      return reinterpret_cast<uint16_t*>(rec + (part == 0 ? REC_TH : part == 1 ? REC_TL : REC_P)) +
             rec_elem(i & 31, 32 + (j & 31));
    };

    // A (strictly lower, scaled) into LDS and P (lower incl. diagonal,
    // scaled) straight to the record: element (i, j) = acc * row factor(i) *
    // n_k,j * exp(G_i - G_j), the exponential (on the hardware base-2
    // exponential of the f64 difference of the base-2 prefixes) and its
    // product with n_k,j shared by the two; a lane's four columns of row i go
    // out as one 16-byte LDS store and one 8-byte record store.  Only the
    // four diagonal tiles need the triangle masks.
    auto ap_tile = [&](auto diag, int k, int t, int ti, int tj) {
      const int i = 16 * ti + cl;
      const int j0 = 16 * tj + 4 * g;
      const double gi = sh.Gd[hs][i];
      const double2 ga = *reinterpret_cast<const double2*>(&sh.Gd[hs][j0]);
      const double2 gb = *reinterpret_cast<const double2*>(&sh.Gd[hs][j0 + 2]);
      const double gj[4] = {ga.x, ga.y, gb.x, gb.y};
      const float rfa = sh.bt[hs][i] * sh.nk[i];
      const float rfp = a.scale * sh.nq[i];
      const float4 c4 = *reinterpret_cast<const float4*>(&sh.nk[j0]);
      const float cj[4] = {c4.x, c4.y, c4.z, c4.w};
      float xa[4], pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ec = __builtin_amdgcn_exp2f((float)(gi - gj[r])) * cj[r];
        xa[r] = accA[k][r] * rfa * ec;
        pv[r] = accP[k][r] * rfp * ec;
        if constexpr (decltype(diag)::value) {
          xa[r] = j0 + r < i ? xa[r] : 0.0f;
          pv[r] = j0 + r <= i ? pv[r] : 0.0f;
        }
      }
      *reinterpret_cast<float4*>(Ab + t * BLK + cl * LDB + 4 * g) =
          make_float4(xa[0], xa[1], xa[2], xa[3]);
      uint16_t ph[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ph[r] = M::enc(pv[r]);
      *reinterpret_cast<uint2*>(Pg + rec_elem(i, j0)) =
          make_uint2(ph[0] | ((uint32_t)ph[1] << 16), ph[2] | ((uint32_t)ph[3] << 16));
      if (plo) {
        uint16_t pl[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pl[r] = M::enc(pv[r] - M::dec(ph[r]));
        *reinterpret_cast<uint2*>(plo_dst(i, j0)) =
            make_uint2(pl[0] | ((uint32_t)pl[1] << 16), pl[2] | ((uint32_t)pl[3] << 16));
      }
    };
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int t = w + 4 * k;
      if (t < 10) {
        const int ti = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
        const int tj = t - (ti * (ti + 1)) / 2;
        if (ti == tj)
          ap_tile(std::true_type{}, k, t, ti, tj);
        else
          ap_tile(std::false_type{}, k, t, ti, tj);
      }
    }
    // P's strictly-upper blocks (0, 1) and (2, 3) reach the walk as zeros
    // without being stored; the low part's, in the free quadrants the walk
    // fetches for an f32 output, are stored as zeros
    if (plo && tid_h < 64) {
      const int blk = tid_h >> 5, e = tid_h & 31;
      const int i = 32 * blk + (e >> 1), j8 = 32 * blk + 16 + 8 * (e & 1);
      *reinterpret_cast<uint4*>(plo_dst(i, j8)) = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();

    // diagonal blocks of T = (I + A)^{-1}: forward substitution, one column per
    // lane, all four blocks on wave 0 (lane group g takes block g), so the
    // other waves leave their SIMDs to the workgroups sharing the CU
    if (w == 0) {
      const float* Ad = Ab + lower_blk(g, g) * BLK;
      const int col = cl;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = (r == col) ? 1.0f : 0.0f;
#pragma unroll
        for (int m = 0; m < r; ++m) v -= Ad[r * LDB + m] * x[m];
        x[r] = v;
        asm volatile("" ::: "memory");  // load row r + 1 of A only now: bounds the live registers
      }
      float* Td = Tb + lower_blk(g, g) * BLK;
#pragma unroll
      for (int r = 0; r < 16; ++r) Td[r * LDB + col] = x[r];
    }
    __syncthreads();

    // off-diagonal blocks, on 16x16x16 products of the f32 MFMA (A: lane
    // (m = l%16, k = l/16), B: lane (k = l/16, n = l%16), D: lane
    // (m = 4 (l/16) + r, n = l%16)), in 32 x 32 halves: with T1, T2 the
    // inverses of the upper-left and lower-right halves and A21 the
    // lower-left half of A, T21 = -T2 A21 T1, so
    //   pass 1: T_10 = -T_11 A_10 T_00 and T_32 = -T_33 A_32 T_22 (two waves),
    //   pass 2: Y = A21 T1, one 16x16 block per wave,
    //   pass 3: T21 = -T2 Y, one block per wave.
    // Partial products go through the waves' slots of R.
    auto mma_blk = [&](const float* X, int ldx, const float* Y, int ldy, f32x4 acc) {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[cl * ldx + 4 * s4 + g],
                                                   Y[(4 * s4 + g) * ldy + cl], acc, 0, 0, 0);
      return acc;
    };
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    float* Rw = sh.u.at.R[w];
    if (w < 2) {
      const int i = 2 * w + 1, j = 2 * w;
      const f32x4 r4 = mma_blk(Ab + lower_blk(i, j) * BLK, LDB, Tb + lower_blk(j, j) * BLK, LDB,
                               zero4);
#pragma unroll
      for (int r = 0; r < 4; ++r) Rw[(4 * g + r) * 17 + cl] = r4[r];
      __builtin_amdgcn_wave_barrier();
      const f32x4 t4 = mma_blk(Tb + lower_blk(i, i) * BLK, LDB, Rw, 17, zero4);
      float* Tij = Tb + lower_blk(i, j) * BLK;
#pragma unroll
      for (int r = 0; r < 4; ++r) Tij[(4 * g + r) * LDB + cl] = -t4[r];
    }
    __syncthreads();
    {
      const int i = 2 + (w >> 1), j = w & 1;
      f32x4 y4 = zero4;
      for (int k = j; k < 2; ++k)
        y4 = mma_blk(Ab + lower_blk(i, k) * BLK, LDB, Tb + lower_blk(k, j) * BLK, LDB, y4);
#pragma unroll
      for (int r = 0; r < 4; ++r) Rw[(4 * g + r) * 17 + cl] = y4[r];
    }
    __syncthreads();
    {
      const int i = 2 + (w >> 1), j = w & 1;
      f32x4 t4 = zero4;
      for (int k = 2; k <= i; ++k)
        t4 = mma_blk(Tb + lower_blk(i, k) * BLK, LDB, sh.u.at.R[2 * (k - 2) + j], 17, t4);
      float* Tij = Tb + lower_blk(i, j) * BLK;
#pragma unroll
      for (int r = 0; r < 4; ++r) Tij[(4 * g + r) * LDB + cl] = -t4[r];
    }
    __syncthreads();

    // T_b = T diag(beta), split into high and low 16-bit parts; only the ten
    // lower blocks are stored (those above the diagonal are zero or the free
    // quadrant)
    uint16_t* Th = reinterpret_cast<uint16_t*>(rec + REC_TH);
    uint16_t* Tl = reinterpret_cast<uint16_t*>(rec + REC_TL);
    // eight consecutive columns of a row per thread: one 16-byte store each
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int idx = tid_h + 256 * k;
      const int i = idx >> 3, j8 = 8 * (idx & 7);
      const int bi = i >> 4, bj = j8 >> 4;
      if (bj > bi) continue;  // zero blocks and the free quadrant
      const float* tr = Tb + lower_blk(bi, bj) * BLK + (i & 15) * LDB + (j8 & 15);
      const float4 t0 = *reinterpret_cast<const float4*>(tr);
      const float4 t1 = *reinterpret_cast<const float4*>(tr + 4);
      const float4 b0 = *reinterpret_cast<const float4*>(&sh.bt[hs][j8]);
      const float4 b1 = *reinterpret_cast<const float4*>(&sh.bt[hs][j8 + 4]);
      const float x[8] = {t0.x * b0.x, t0.y * b0.y, t0.z * b0.z, t0.w * b0.w,
                          t1.x * b1.x, t1.y * b1.y, t1.z * b1.z, t1.w * b1.w};
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t h0 = M::enc(x[2 * e]), h1 = M::enc(x[2 * e + 1]);
        const uint16_t l0 = M::enc(x[2 * e] - M::dec(h0)), l1 = M::enc(x[2 * e + 1] - M::dec(h1));
        hw[e] = h0 | ((uint32_t)h1 << 16);
        lw[e] = l0 | ((uint32_t)l1 << 16);
      }
      *reinterpret_cast<uint4*>(Th + rec_elem(i, j8)) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4*>(Tl + rec_elem(i, j8)) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    __syncthreads();  // the next head rewrites A and T (and, per group, Gd and bt)
  }
}

// Launch part of the prep that also forms the metadata (one stream order, at
// most 256 sequences): workgroup 0 runs the metadata kernel's work in the
// prep's LDS, and every other workgroup finds its (sequence, chunk), in
// sequence order, from cu_seqlens itself -- so no launch waits for the
// metadata before the walks.
constexpr int kPartSelf = 3;
constexpr int kSelfMaxSeqs = 256;

struct MetaIn {
  int ntiles, ncu, ksmax, smax;
};

// One workgroup per (chunk, q/k head) unit of one launch part, the chunks
// taken in rank order (longest sequences first; in sequence order for
// kPartSelf); the grid covers every chunk the call can have, and workgroups
// past the part's units leave at once.
template <int TIN, bool SELF>
__global__ __launch_bounds__(256, 4) void chunk_prep_kernel(PrefillArgs a, MetaPtrs m,
                                                            char* recs, int part, MetaIn mi) {
  __shared__ __align__(16) PrepLds sh;
  const int n = (int)a.num_seqs;
  // records the workspace holds: a well-formed cu_seqlens never needs more,
  // but overlapping ranges (clamped, not rejected) can, and their surplus
  // records are not formed (the walk does not read past this count either)
  const int64_t rec_cap = (a.total_tokens + CK - 1) / CK + a.num_seqs;
  if constexpr (SELF) {  // part == kPartSelf
    static_assert(sizeof(MetaLds) <= sizeof(PrepLds), "the metadata's LDS inside the prep's");
    if (blockIdx.x == 0) {
      meta_body(a, m, mi.ntiles, mi.ncu, 0, mi.ksmax, mi.smax, *reinterpret_cast<MetaLds*>(&sh));
      return;
    }
    __shared__ int32_t scan_part[4];
    __shared__ int32_t found[2];
    const int64_t u = blockIdx.x - 1;
    const int cr = (int)(u / a.hk);  // chunk index in sequence order: the record's
    const int hk = (int)(u % a.hk);
    const int t = threadIdx.x;
    int32_t c = 0;
    if (t < n) {
      int64_t t0, t1;
      chunk_bounds(a, t, t0, t1);
      c = (int32_t)((t1 - t0 + CK - 1) / CK);
    }
    if (t == 0) found[0] = -1;
    const int32_t incl = block_scan256(c, scan_part);  // its barriers order the line above
    if (t < n && cr >= incl - c && cr < incl) {
      found[0] = t;
      found[1] = cr - (incl - c);
    }
    __syncthreads();
    const int s = found[0];
    // past the call's last chunk, or past the records the workspace holds
    // (the same for the whole workgroup)
    if (s < 0 || cr >= rec_cap) return;
    const int j = found[1];
    int64_t t0, t1;
    chunk_bounds(a, s, t0, t1);
    const int64_t tb = t0 + (int64_t)j * CK;
    prep_unit<TIN>(a, recs, sh, cr, hk, tb, (int)min((int64_t)CK, t1 - tb));
  } else {
    (void)mi;
    int c0, c1;
    part_chunks(m, n, part, c0, c1);
    const int64_t u = blockIdx.x;
    if (u >= (int64_t)(c1 - c0) * a.hk) return;
    const int cr = c0 + (int)(u / a.hk);
    const int hk = (int)(u % a.hk);
    int lo = 0, hi = n - 1;  // largest rank r with ocs[r] <= cr
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (m.ocs[mid] <= cr) lo = mid; else hi = mid - 1;
    }
    const int s = m.order[lo];
    const int j = cr - m.ocs[lo];
    if (m.cs[s] + j >= rec_cap) return;  // only with overlapping ranges
    int64_t t0, t1;
    chunk_bounds(a, s, t0, t1);
    const int64_t tb = t0 + (int64_t)j * CK;
    const int L = (int)min((int64_t)CK, t1 - tb);
    prep_unit<TIN>(a, recs, sh, m.cs[s] + j, hk, tb, L);
  }
}

// ---------------------------------------------------------------------------
// the state walk
// ---------------------------------------------------------------------------
// One workgroup of NW waves walks one (sequence, v-head, block of 16 NW state
// rows); wave w owns the 16 state rows dv = dv0 + 16 w .. +15 for all 128 keys
// and keeps them transposed, St = S^T [dk][dv], in eight MFMA accumulator
// tiles.  Every product of a chunk step takes its state operand straight from
// those registers and every result's accumulator layout is the B-operand
// layout of the product that consumes it, so the waves never exchange data:
// they share only the chunk's inputs, staged once per workgroup in LDS.  A
// further wave (the load wave) stages them: while the compute waves work on
// chunk ch it brings chunk ch + 1 into the other of two LDS buffers, so no
// compute wave issues a global load or waits behind a full load queue (under
// a busy memory system that stall took about a tenth of a chunk step).
//
// MFMA 16x16x32 layouts (lane l, g = l / 16, c = l % 16):
//   A: A[c][8g + e] (e < 8),  B: B[8g + e][c],  D: D[4g + r][c] (r < 4).
// Two D tiles stacked along k form one B operand when row m of tile 2j + h
// stands for index 32j + 8 (m / 4) + 4h + m % 4: lane group g then holds the
// 8 consecutive indices 32j + 8g .. +7, the standard B layout.  The token
// blocks of a chunk and the key blocks of St are both numbered that way.
__device__ __forceinline__ int blk_row(int b, int m) {
  return 32 * (b >> 1) + 8 * (m >> 2) + 4 * (b & 1) + (m & 3);
}

// LDS layouts of the chunk operands.  On gfx950 a 16-byte LDS read serves 16
// lanes per cycle -- lane quads {0, 3, 5, 6} or {1, 2, 4, 7} of a 32-lane half
// -- and an 8- or 2-byte access 32 lanes; lanes of one cycle must touch
// distinct banks (4 bytes each, 64 banks).  The 16-byte chunks of a row are
// XOR-swizzled by row so that the operand reads are conflict-free:
//   K and Q, [token][key]: 16 chunks per row, swizzle 4 (row % 4) + beta(row / 8 % 4);
//   T_b and P, [token][token]: 8 chunks per row, swizzle 4 (row / 2 % 2) + beta(row / 8 % 4);
// with beta a permutation of 0..3 that spreads the two lane groups of a cycle.
__device__ __forceinline__ int swz_beta(int q) { return (0x1320 >> (4 * q)) & 3; }
__device__ __forceinline__ int kq_swz(int row) { return 4 * (row & 3) + swz_beta((row >> 3) & 3); }
__device__ __forceinline__ int tp_swz(int row) {
  return 4 * ((row >> 1) & 1) + swz_beta((row >> 3) & 3);
}

constexpr uint32_t kBufferFlags = 0x00020000;  // raw buffer resource word 3 on gfx9
// a buffer offset past every output range of the walk (chunks of rows stay below 2^30 bytes)
constexpr int kDropOffset = 1 << 30;

// V of the chunk, [token][columns] 16-bit, 16-byte chunks XOR-swizzled so the
// four rows 8 apart read by one D-layout access hit distinct banks
__device__ __forceinline__ int v_swz(int row) { return ((row >> 3) & 3) << 1; }

// One chunk's inputs in LDS for a workgroup of NW waves with NB 16-column
// blocks each.  The walk keeps two and fills one with direct global-to-LDS
// loads while it computes on the other.
template <int NW, int NB>
struct WalkBuf {
  static constexpr int VC = 16 * NW * NB;  // state rows (V columns) of the workgroup
  uint16_t K[CK * DKC], Q[CK * DKC];
  uint16_t Th[CK * CK], Tl[CK * CK], P[CK * CK];
  uint16_t V[CK * VC];
  float F[4 * CK];
};

struct WalkCtx {
  const PrefillArgs* a;
  const char* recs;
  int64_t t_begin, t_end;
  int c0, h, hk, dv0;
  int v_on;  // 0: v reads as zeros (the identity's walk)
};

__device__ __forceinline__ int chunk_len(const WalkCtx& c, int ch) {
  return (int)min((int64_t)CK, c.t_end - (c.t_begin + (int64_t)ch * CK));
}

__device__ __forceinline__ const char* chunk_rec(const WalkCtx& c, int ch) {
  return c.recs + ((int64_t)(c.c0 + ch) * c.a->hv + c.h) * REC_BYTES;
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at dst + 16 l (dst is the same for the whole wave).
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}

// The same through a buffer resource: a lane whose offset lies past the
// resource's range reads zeros.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, int off, void* dst) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, off, 0, 0, 0);
}

// Per-lane byte offsets, within a chunk, of the 16-byte units a lane loads:
// each 1 KB wave load covers 64 consecutive units of a matrix in LDS, unit p
// holding the row's chunk that the swizzle puts there.
template <int NW, int NB>
struct StageOffsets {
  static constexpr int NKQ = 16 / NW;      // wave loads of K (and of Q) per wave
  static constexpr int NTP = 8 / NW;       // of T_b hi, T_b lo and P
  static constexpr int NVL = 2 * NB;       // of V
  int k[NKQ], q[NKQ], tp[NTP], v[NVL];
};

template <int NW, int NB, bool FULL>
__device__ __forceinline__ void stage_offsets(StageOffsets<NW, NB>& o, const PrefillArgs& a,
                                              int dv0, int w, int lane) {
  using SO = StageOffsets<NW, NB>;
#pragma unroll
  for (int i = 0; i < SO::NKQ; ++i) {
    const int p = 64 * (NW * i + w) + lane, row = p >> 4;
    const int chg = (p & 15) ^ kq_swz(row);
    o.k[i] = (int)(row * a.k_rs * 2) + 16 * chg;
    o.q[i] = (int)(row * a.q_rs * 2) + 16 * chg;
  }
#pragma unroll
  for (int i = 0; i < SO::NTP; ++i) {
    const int p = 64 * (NW * i + w) + lane, row = p >> 3, chunk = (p & 7) ^ tp_swz(row);
    // the free upper-right quadrants hold P's low part for an f32 output and
    // are otherwise not fetched, nor are the zero blocks (0, 1) and (2, 3):
    // their offset then lies past the record and they arrive as zeros
    const bool free_q = row < 32 && chunk >= 4;
    const bool zero_blk = (chunk >> 1) > (row >> 4) && !free_q;
    o.tp[i] = (!FULL && free_q) || zero_blk ? kDropOffset : 2 * rec_elem(row, 8 * chunk);
  }
  constexpr int VCH = 2 * NW * NB;  // 16-byte chunks per V row
#pragma unroll
  for (int i = 0; i < SO::NVL; ++i) {
    const int p = 64 * (NW * i + w) + lane, row = p / VCH;
    const int chg = (p % VCH) ^ v_swz(row);
    // columns past dv (a partial last block) re-read the last 8 columns
    o.v[i] = (int)(row * a.v_rs * 2) + 2 * min(dv0 + 8 * chg, a.dv - 8);
  }
}

// Issues part PART of the loads of chunk `ch` into B: 0 = K, 1 = Q, 2 = T_b
// high/low and P, 3 = the V columns and the factors.  The q/k/v rows go
// through buffer resources that end at the chunk's last token, so rows past
// the end of the sequence arrive as zeros.  Issued by the walk's load wave,
// one call per compute wave's share.  A walk without outputs (OUTS false)
// loads neither Q nor P.
template <int NW, int NB, int PART, bool OUTS>
__device__ __forceinline__ void stage_dma_part(WalkBuf<NW, NB>& B, const WalkCtx& c, int ch,
                                               int w, int lane, const StageOffsets<NW, NB>& o) {
  using SO = StageOffsets<NW, NB>;
  const PrefillArgs& a = *c.a;
  const int64_t tb = c.t_begin + (int64_t)ch * CK;
  const int L = chunk_len(c, ch);
  if constexpr (PART == 0) {
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(static_cast<const uint16_t*>(a.k) + tb * a.k_rs +
                              (int64_t)c.hk * DKC),
        0, (int)(L * a.k_rs * 2), kBufferFlags);
#pragma unroll
    for (int i = 0; i < SO::NKQ; ++i) dma16_buf(kr, o.k[i], B.K + 512 * (NW * i + w));
  } else if constexpr (PART == 1) {
    if constexpr (!OUTS) return;
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(static_cast<const uint16_t*>(a.q) + tb * a.q_rs +
                              (int64_t)c.hk * DKC),
        0, (int)(L * a.q_rs * 2), kBufferFlags);
#pragma unroll
    for (int i = 0; i < SO::NKQ; ++i) dma16_buf(qr, o.q[i], B.Q + 512 * (NW * i + w));
  } else if constexpr (PART == 2) {
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(chunk_rec(c, ch)), 0, REC_BYTES, kBufferFlags);
#pragma unroll
    for (int i = 0; i < SO::NTP; ++i) {
      const int u = NW * i + w;
      dma16_buf(rr, REC_TH + o.tp[i], B.Th + 512 * u);
      dma16_buf(rr, REC_TL + o.tp[i], B.Tl + 512 * u);
      if constexpr (OUTS) dma16_buf(rr, REC_P + o.tp[i], B.P + 512 * u);
    }
  } else {
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(static_cast<const uint16_t*>(a.v) + tb * a.v_rs +
                              (int64_t)c.h * a.dv),
        0, c.v_on ? (int)(L * a.v_rs * 2) : 0, kBufferFlags);
#pragma unroll
    for (int i = 0; i < SO::NVL; ++i) dma16_buf(vr, o.v[i], B.V + 512 * (NW * i + w));
    if (w == 0) dma16(chunk_rec(c, ch) + REC_F + 16 * lane, B.F);
  }
}

// All loads of chunk `ch` into B.
template <int NW, int NB, bool OUTS>
__device__ __forceinline__ void stage_dma(WalkBuf<NW, NB>& B, const WalkCtx& c, int ch, int w,
                                          int lane, const StageOffsets<NW, NB>& o) {
  stage_dma_part<NW, NB, 0, OUTS>(B, c, ch, w, lane, o);
  stage_dma_part<NW, NB, 1, OUTS>(B, c, ch, w, lane, o);
  stage_dma_part<NW, NB, 2, OUTS>(B, c, ch, w, lane, o);
  stage_dma_part<NW, NB, 3, OUTS>(B, c, ch, w, lane, o);
}

// Output element encoding of the state walk.
template <int TOUT>
struct OutT {
  typedef uint16_t type;
  static __device__ __forceinline__ uint16_t enc(float x) {
    return TOUT == kBF16 ? f32_to_bf16(x) : f32_to_f16(x);
  }
};
template <>
struct OutT<kF32> {
  typedef float type;
};
typedef __fp16 lds_h4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// 8-byte transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, result lane i element e is element i % 4 of the 8 bytes addressed by
// lane 4e + i / 4 of the group.
__device__ __forceinline__ u16x4 lds_read_tr(const uint16_t* p) {
  typedef __attribute__((address_space(3))) lds_h4 lds_ptr_t;
  const lds_h4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_ptr_t*)(p));
  return __builtin_bit_cast(u16x4, v);
}

// Packs two D tiles (tile 2j: slots 0-3, tile 2j + 1: slots 4-7) into a B
// operand, rounded to 16 bits.
typedef float f32x8 __attribute__((ext_vector_type(8)));
template <int TIN>
__device__ __forceinline__ void pack_hi(const f32x4& t0, const f32x4& t1,
                                        typename MT<TIN>::x8& hi) {
  const f32x8 x = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
  hi = __builtin_convertvector(x, typename MT<TIN>::x8);
}

// The same split into 16-bit high and low parts (lo = x - hi, rounded).
template <int TIN>
__device__ __forceinline__ void pack_split(const f32x4& t0, const f32x4& t1,
                                           typename MT<TIN>::x8& hi, typename MT<TIN>::x8& lo) {
  using x8 = typename MT<TIN>::x8;
  const f32x8 x = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
  hi = __builtin_convertvector(x, x8);
  if constexpr (TIN == kF16) {
    // x - hi as one mixed-precision FMA per element, the f16 half of the
    // packed pair widened inside the instruction (v_fma_mix_f32): exact, as
    // the subtraction is, and one instruction instead of a convert and a
    // subtraction (the compiler turns a plain fma with -1 back into those)
    const u32x4 hw = __builtin_bit_cast(u32x4, hi);
    f32x8 d;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float d0, d1;
      asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(d0) : "v"(hw[i]), "v"(x[2 * i]));
      asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
          : "=v"(d1) : "v"(hw[i]), "v"(x[2 * i + 1]));
      d[2 * i] = d0;
      d[2 * i + 1] = d1;
    }
    lo = __builtin_convertvector(d, x8);
  } else {
    lo = __builtin_convertvector(x - __builtin_convertvector(hi, f32x8), x8);
  }
}

// What a walk workgroup does (see the segment notes at the metadata):
enum WalkKind {
  kFullWalk = 0,  // a sequence or one of its segments, with outputs
  kWalkA0 = 1,    // segment 0 of a split sequence, state only: S_in of segment 1
  kWalkLoc = 2,   // a middle segment from zero, state only: its S_loc
  kWalkTrn = 3    // a middle segment from the identity with v = 0 (Dk rows): its M
};

// Outputs leave through a buffer resource whose range ends at the chunk's last
// row: stores of rows past the end of the sequence (and of a block past dv)
// fall outside it and are dropped by the hardware, with no branch per row.
// OUTS: the walk forms outputs (full walks); else it updates the state alone
// (the first phase of split sequences) and never loads Q or P.
template <int TIN, int TOUT, int NW, int NB, int MINB, bool OUTS>
__global__ __launch_bounds__(64 * (NW + 1), MINB) void chunk_state_kernel(
    PrefillArgs a, MetaPtrs m, const char* recs, float* segws, int seg_slots, int ntiles,
    int max_chunks, int part) {
  constexpr int NTH = 64 * (NW + 1);  // the compute waves and the load wave
  constexpr int NTHC = 64 * NW;       // the compute waves
  constexpr int VC = WalkBuf<NW, NB>::VC;
  // the two chunk buffers are dynamic LDS: the static size would make the
  // compiler assume one workgroup per CU and spread the registers over the
  // accumulation file, costing a copy for every accumulator the VALU touches
  extern __shared__ __align__(16) char walk_lds[];
  WalkBuf<NW, NB>* sb = reinterpret_cast<WalkBuf<NW, NB>*>(walk_lds);
  using M = MT<TIN>;
  using x8 = typename M::x8;
  // The state's history term Q S^T always takes the high and low parts of S:
  // with the high part only, an output row whose terms nearly cancel (a few
  // in 10^5 at T = 4096) lost up to 2e-2 of its size, ten times a bf16
  // rounding.  The in-chunk term P U takes the high parts of P and U for a
  // 16-bit output (a row of it errs by about one 16-bit rounding), the full
  // high/low products for an f32 output.
  constexpr bool kFullOut = TOUT == kF32;

  // XCD-aware mapping.  Workgroups are dealt round-robin to the 8 XCDs, each
  // with its own L2; the tiles of one v-head re-read the same per-chunk
  // records, and the v-heads of one GQA group the same q/k rows, so a unit
  // (walk item, q/k head) keeps all ratio * ntiles of its workgroups on one
  // XCD: block b -> xcd = b % 8, unit = (b / 8) / per_unit * 8 + xcd.
  const int ratio = a.hv / a.hk;
  const int per_unit = ratio * ntiles;
  const int xcd = blockIdx.x % kXcds;
  const int rblk = blockIdx.x / kXcds;
  const int unit = (rblk / per_unit) * kXcds + xcd;
  const int item = unit / a.hk;
  const int n = (int)a.num_seqs;
  const int ksplit = m.info[0], ks = m.info[1], nseg_split = m.info[2];
  // this launch's walk items
  int rank, seg, nseg, kind;
  if constexpr (!OUTS) {
    // phase A of the split ranks [0, ks): per rank 2 S - 3 items: segment 0,
    // then (S_loc, M) of each middle segment 1 .. S - 2
    const int per = 2 * nseg_split - 3;
    if (ks == 0 || per <= 0) return;
    rank = item / per;
    if (rank >= ks) return;
    const int li = item % per;
    seg = li == 0 ? 0 : 1 + (li - 1) / 2;
    kind = li == 0 ? kWalkA0 : ((li - 1) & 1) ? kWalkTrn : kWalkLoc;
    nseg = nseg_split;
  } else {
    // ranks of this launch part: 0 = [0, k), 1 = [k, n), 2 = all; the split
    // ranks among them (always the first) have one item per segment
    const int r0 = part == 1 ? ksplit : 0, r1 = part == 0 ? ksplit : n;
    const int nsplit = max(0, min(ks, r1) - r0);
    if (item < nsplit * nseg_split) {
      rank = r0 + item / nseg_split;
      seg = item % nseg_split;
      nseg = nseg_split;
    } else {
      rank = r0 + nsplit + (item - nsplit * nseg_split);
      seg = 0;
      nseg = 1;
    }
    if (rank >= r1) return;
    kind = kFullWalk;
  }
  // state rows of this walk: dv, or Dk for the identity's walk
  const int rows = kind == kWalkTrn ? DKC : a.dv;
  const int j0 = rblk % per_unit;
  const int tile = j0 % ntiles;
  if (tile * VC >= rows) return;
  const int h = (unit % a.hk) * ratio + j0 / ntiles;
  const int s = m.order[rank];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 4, cl = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  WalkCtx c;
  c.a = &a;
  c.recs = recs;
  int64_t seq_t0, seq_t1;
  chunk_bounds(a, s, seq_t0, seq_t1);
  // a well-formed cu_seqlens gives cs[s] + chunks <= max_chunks; a malformed
  // one (overlapping ranges) must still never index past the workspace
  const int nch_seq =
      max(0, min((int)((seq_t1 - seq_t0 + CK - 1) / CK), max_chunks - m.cs[s]));
  const int seg_len = nseg > 1 ? m.info[3 + rank] : nch_seq;
  const int ch0 = min(seg * seg_len, nch_seq);
  const int nch = min(seg_len, nch_seq - ch0);
  c.t_begin = seq_t0 + (int64_t)ch0 * CK;
  c.t_end = min(seq_t1, seq_t0 + (int64_t)(ch0 + nch) * CK);
  c.c0 = m.cs[s] + ch0;
  c.h = h;
  c.hk = h / ratio;
  c.dv0 = tile * VC;
  c.v_on = kind == kWalkTrn ? 0 : 1;
  // this wave's blocks: state rows dvw + 16 nb .. +15
  const int dvw = c.dv0 + 16 * NB * w;
  const int64_t slot = a.idx ? (int64_t)a.idx[s] : (int64_t)s;
  const int64_t out_rs = (int64_t)a.hv * a.dv;

  if (slot < 0 || slot >= a.num_slots) {
    // caller error: NaN outputs for these rows, no state access
    if constexpr (OUTS) {
      for (int64_t t = c.t_begin + tid / VC; t < c.t_end; t += NTH / VC) {
        const int col = c.dv0 + tid % VC;
        if (col < a.dv) store1(a.out, a.out_dt, t * out_rs + (int64_t)h * a.dv + col,
                               __builtin_nanf(""));
      }
    }
    return;
  }

  // The load wave (the workgroup's last) issues every chunk's loads into LDS
  // and waits for them, so no compute wave ever stalls behind a full load
  // queue; it meets the compute waves at each of their barriers (two per
  // folded segment, one after clearing the buffers, one per chunk).
  if (w == NW) {
    if (kind == kFullWalk)
      for (int i = 1; i < seg; ++i) {
        lds_barrier();
        lds_barrier();
      }
    if (nch == 0) return;
    StageOffsets<NW, NB> sos[NW];
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) stage_offsets<NW, NB, kFullOut>(sos[ww], a, c.dv0, ww, lane);
    lds_barrier();  // both buffers cleared
    for (int ch = 0; ch <= nch; ++ch) {
      // chunk 0 before the first step, chunk ch + 1 during step ch; the
      // buffer it fills was released at the barrier that ended step ch - 1
      if (ch < nch) {
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) stage_dma<NW, NB, OUTS>(sb[ch & 1], c, ch, ww, lane, sos[ww]);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
    }
    return;
  }
  const bool init = a.has_init ? a.has_init[s] != 0 : true;
  const int64_t Sg = ((slot * a.hv + h) * a.dv + dvw + cl) * DKC;  // element offset in the pool
  using Ot = typename OutT<TOUT>::type;
  Ot* out = static_cast<Ot*>(a.out) + (int64_t)h * a.dv + dvw;  // this wave's column 0

  // The split sequence's workspace states: slot 0 its initial state, 1 the
  // entry state of segment 1, 2 i and 2 i + 1 the S_loc and M^T of middle
  // segment i.  One state is ntiles tiles of VC rows x Dk f32, each kept in the
  // walk's register layout (16 bytes per lane and tile, a wave's lanes
  // contiguous); M^T alone is a plain [Dk][Dk] row-major matrix.
  constexpr int kTileFloats = NB * 8 * NW * 64 * 4;
  const size_t slot_floats = (size_t)ntiles * kTileFloats;
  auto ws_state = [&](int sl) {
    return segws + ((size_t)(rank * a.hv + h) * seg_slots + sl) * slot_floats;
  };
  auto tile_off = [&](int nb, int kb) { return (((nb * 8 + kb) * NW + w) * 64 + lane) * 4; };

  // St[nb][kb], element r: S[dvw + 16 nb + cl][blk_row(kb, 4g + r)]
  f32x4 St[NB][8];
  auto ld_tiles = [&](const float* p) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        St[nb][kb] = *reinterpret_cast<const f32x4*>(p + tile * kTileFloats + tile_off(nb, kb));
  };
  auto st_tiles = [&](float* p) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        *reinterpret_cast<f32x4*>(p + tile * kTileFloats + tile_off(nb, kb)) = St[nb][kb];
  };
  const bool from_pool = kind == kWalkA0 || (kind == kFullWalk && nseg == 1);
  if (from_pool || kind == kWalkLoc || (kind == kFullWalk && seg == 0)) {
    // the real initial state (from the pool, or as segment 0 of a split
    // sequence from the copy its phase-A walk kept: the last segment may
    // already be overwriting the pool slot), or zeros
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bool ld = init && kind != kWalkLoc && dvw + 16 * nb < rows;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ld && from_pool) {
          v = state_load4_rt(a.state_dt, a.pool, Sg + 16 * nb * DKC + blk_row(kb, 4 * g));
        } else if (ld) {
          const f32x4 t = *reinterpret_cast<const f32x4*>(ws_state(0) + tile * kTileFloats +
                                                          tile_off(nb, kb));
          v = make_float4(t[0], t[1], t[2], t[3]);
        }
        St[nb][kb] = (f32x4){v.x, v.y, v.z, v.w};
      }
    }
    if (kind == kWalkA0 && init) st_tiles(ws_state(0));
  } else if (kind == kWalkTrn) {
    // the identity: S[row][key] = 1 where key == row
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          St[nb][kb][r] = blk_row(kb, 4 * g + r) == dvw + 16 * nb + cl ? 1.0f : 0.0f;
  } else {
    ld_tiles(ws_state(1));  // segment j >= 1 starts from the entry state of segment 1 ...
  }
  auto store_state = [&]() {
    if (kind == kFullWalk) {
      if (seg != nseg - 1) return;  // only the last segment's final state is kept
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (dvw + 16 * nb < a.dv) {
#pragma unroll
          for (int kb = 0; kb < 8; ++kb)
            state_store4_rt(a.state_dt, a.pool, Sg + 16 * nb * DKC + blk_row(kb, 4 * g),
                            make_float4(St[nb][kb][0], St[nb][kb][1], St[nb][kb][2],
                                        St[nb][kb][3]));
        }
      }
    } else if (kind == kWalkTrn) {
      // M^T[key][row] = S[row][key]: a plain row-major [Dk][Dk] matrix
      float* mt = ws_state(2 * seg + 1);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            mt[blk_row(kb, 4 * g + r) * DKC + dvw + 16 * nb + cl] = St[nb][kb][r];
    } else {
      st_tiles(ws_state(kind == kWalkA0 ? 1 : 2 * seg));
    }
  };

  // Per-lane LDS offsets (elements).  Every operand row of token block b is
  // blk_row(b, m) = 32 (b / 2) + 4 (b % 2) + rm with rm = 8 (m / 4) + m % 4, and
  // the swizzles depend on rm only, so each read is a per-lane base (one per
  // k-step) plus a compile-time offset for the block.
  const int rmA = 8 * (cl >> 2) + (cl & 3);  // A-operand row within a block pair
  const int sK = kq_swz(rmA);                  // the swizzles of those rows (any block)
  const int sT = tp_swz(rmA);
  int kqb[4], tpb[2], trb[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) kqb[jj] = rmA * DKC + 8 * ((4 * jj + g) ^ sK);
#pragma unroll
  for (int j = 0; j < 2; ++j) tpb[j] = rmA * CK + 8 * ((4 * j + g) ^ sT);

  if (kind == kFullWalk && seg > 0) {
    // ... and folds in middle segments 1 .. seg - 1: S <- S M_i + S_loc,i, as
    // St <- M_i^T St + S_loc,i^T.  M_i^T is staged in LDS as 16-bit high / low
    // parts with K's row layout and swizzle (Dk rows, 8 row blocks), and each
    // product is the X = K St product with M_i^T in K's place.
    uint16_t* mh = reinterpret_cast<uint16_t*>(walk_lds);
    uint16_t* ml = mh + DKC * DKC;
    for (int i = 1; i < seg; ++i) {
      const float* mt = ws_state(2 * i + 1);
      for (int u = tid; u < DKC * 16; u += NTHC) {
        const int row = u >> 4, c8 = u & 15;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(mt + row * DKC + 8 * c8);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(mt + row * DKC + 8 * c8 + 4);
        x8 hi, lo;
        pack_split<TIN>(x0, x1, hi, lo);
        const int off = row * DKC + 8 * (c8 ^ kq_swz(row));
        *reinterpret_cast<x8*>(mh + off) = hi;
        *reinterpret_cast<x8*>(ml + off) = lo;
      }
      lds_barrier();
      f32x4 Sn[NB][8];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) Sn[nb][kb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          x8 sh, sl;
          pack_split<TIN>(St[nb][2 * jj], St[nb][2 * jj + 1], sh, sl);
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) {
            const int rb = 32 * (kb >> 1) + 4 * (kb & 1);
            const x8 ah = *reinterpret_cast<const x8*>(mh + kqb[jj] + rb * DKC);
            const x8 al = *reinterpret_cast<const x8*>(ml + kqb[jj] + rb * DKC);
            Sn[nb][kb] = M::mma(ah, sh, Sn[nb][kb]);
            Sn[nb][kb] = M::mma(ah, sl, Sn[nb][kb]);
            Sn[nb][kb] = M::mma(al, sh, Sn[nb][kb]);
          }
        }
      }
      const float* sloc = ws_state(2 * i);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
          St[nb][kb] = Sn[nb][kb] +
                       *reinterpret_cast<const f32x4*>(sloc + tile * kTileFloats + tile_off(nb, kb));
      lds_barrier();  // every wave is done with M_i^T before it is overwritten
    }
  }
  if (nch == 0) {  // no tokens in this walk: the state passes through (or is zeroed)
    store_state();
    return;
  }

  // rows past the end of a sequence arrive as zeros; clearing both buffers
  // first also keeps every row that the first chunk does not load finite
  {
    u32x4* z = reinterpret_cast<u32x4*>(walk_lds);
    constexpr int n16 = (int)(2 * sizeof(WalkBuf<NW, NB>) / 16);
    for (int i = tid; i < n16; i += NTHC) z[i] = (u32x4){0u, 0u, 0u, 0u};
  }
  lds_barrier();
  lds_barrier();  // the load wave has chunk 0 in buffer 0

  {
    // transposing reads: this lane supplies row 32 j + 8 g + 4 h + e, chunk
    // 4 (kb / 2) + q (+ 4 elements when kb is odd); the row swizzle is kq_swz(8 g + e)
    const int e = cl >> 2, q = lane & 3;
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) trb[kp] = (8 * g + e) * DKC + 8 * ((4 * kp + q) ^ kq_swz(8 * g + e));
  }
  // V rows 8 g + ..., column 16 (NB w + nb) + cl of the workgroup (row swizzle 2 g)
  int vb[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    vb[nb] = 8 * g * VC + 8 * ((2 * (NB * w + nb) + (cl >> 3)) ^ (2 * g)) + (cl & 7);
  const int fb = 8 * g;  // factor rows 8 g + ...
  // output element (row 8 g + i, column 16 nb + cl) of a chunk, in bytes
  const int out_lane = (int)((8 * g * out_rs + cl) * (int64_t)sizeof(Ot));
  const int out_row = (int)(out_rs * (int64_t)sizeof(Ot));
  // 16-bit outputs leave as rows: lane l writes row l, 8 columns per 16 bytes
  const int orow_off = lane * out_row;
  int orow_lds[2 * NB];
#pragma unroll
  for (int k = 0; k < 2 * NB; ++k) orow_lds[k] = lane * VC + 8 * ((2 * NB * w + k) ^ v_swz(lane));
  // a block past dv stores at offsets beyond any chunk's range (dropped)
  int blk_off[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) blk_off[nb] = dvw + 16 * nb < a.dv ? 0 : kDropOffset;

  // 16-bit outputs of a chunk are staged as rows in the wave's own columns of
  // that chunk's V space and leave at the end of the step, 16 bytes per lane.
  auto store_rows = [&](const WalkBuf<NW, NB>* __restrict__ buf, int chp) {
    if constexpr (OUTS && TOUT != kF32) {
      const int64_t tbp = c.t_begin + (int64_t)chp * CK;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          out + tbp * out_rs, 0, chunk_len(c, chp) * out_row, kBufferFlags);
      u32x4 row8[2 * NB];
#pragma unroll
      for (int k = 0; k < 2 * NB; ++k) row8[k] = *reinterpret_cast<const u32x4*>(buf->V + orow_lds[k]);
#pragma unroll
      for (int k = 0; k < 2 * NB; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(row8[k], rs, orow_off + 16 * k + blk_off[k >> 1], 0, 0);
    }
  };

  // One chunk step: `cur` holds chunk ch while the load wave fills the other
  // buffer with chunk ch + 1.
  auto chunk_step = [&](WalkBuf<NW, NB>* __restrict__ cur, int ch) {
    const int64_t tb = c.t_begin + (int64_t)ch * CK;
    const int L = chunk_len(c, ch);
    WalkBuf<NW, NB>& sm = *cur;
    // rows [0, L) of this chunk
    const __amdgpu_buffer_rsrc_t orsrc =
        __builtin_amdgcn_make_buffer_rsrc(out + tb * out_rs, 0, L * out_row, kBufferFlags);
    int lane_off = out_lane;
    asm volatile("" : "+v"(lane_off));  // keep the row offsets below out of the loop preheader

    // ---- X = K St and QS = Q St (entry state), St split into B operands on the fly ----
    f32x4 X[NB][4], QS[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        X[nb][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
        QS[nb][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
    // operand fragments of k-step jj + 1 are read while k-step jj multiplies
    x8 kf[2][4], qf[2][4];
    auto read_kq = [&](x8 (&kd)[4], x8 (&qd)[4], int jj) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int rb = 32 * (b >> 1) + 4 * (b & 1);
        kd[b] = *reinterpret_cast<const x8*>(sm.K + kqb[jj] + rb * DKC);
        if constexpr (OUTS) qd[b] = *reinterpret_cast<const x8*>(sm.Q + kqb[jj] + rb * DKC);
      }
    };
    read_kq(kf[0], qf[0], 0);
    // Operands that do not depend on this step's products are read from LDS
    // well ahead of their use, so their latency hides under the MFMAs before
    // them: in the last k-step (which reads no K or Q) the V values and fz
    // factors of Z, and e^{G_C}.
    uint16_t vraw[NB][4][4];
    float4 fz4[4];
    float gc;
    auto read_vz = [&]() {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int rb = 32 * (b >> 1) + 4 * (b & 1);
        fz4[b] = *reinterpret_cast<const float4*>(sm.F + fb + rb);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r) vraw[nb][b][r] = sm.V[vb[nb] + (rb + r) * VC];
      }
      gc = sm.F[3 * CK];
    };
    // St's high/low split of k-step jj + 1 is formed while k-step jj multiplies
    x8 sh[2][NB], sl[2][NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) pack_split<TIN>(St[nb][0], St[nb][1], sh[0][nb], sl[0][nb]);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if (jj < 3) read_kq(kf[(jj + 1) & 1], qf[(jj + 1) & 1], jj + 1);
      else read_vz();
      // the reads above stay a whole k-step ahead of their use: the scheduler
      // would otherwise pull them down next to their MFMAs and wait on each
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const x8 h = sh[jj & 1][nb], l = sl[jj & 1][nb];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          X[nb][b] = M::mma(kf[jj & 1][b], h, X[nb][b]);
          if constexpr (OUTS) QS[nb][b] = M::mma(qf[jj & 1][b], h, QS[nb][b]);
          X[nb][b] = M::mma(kf[jj & 1][b], l, X[nb][b]);
          if constexpr (OUTS) QS[nb][b] = M::mma(qf[jj & 1][b], l, QS[nb][b]);
        }
        if (jj < 3)
          pack_split<TIN>(St[nb][2 * jj + 2], St[nb][2 * jj + 3], sh[(jj + 1) & 1][nb],
                          sl[(jj + 1) & 1][nb]);
      }
    }

    // T_b fragments of U (token blocks b, j <= b / 2) and the fw factors, read
    // while the last products of X finish
    x8 thf[4][2], tlf[4][2];
    float4 fw4[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int rb = 32 * (b >> 1) + 4 * (b & 1);
#pragma unroll
      for (int j = 0; j <= (b >> 1); ++j) {
        thf[b][j] = *reinterpret_cast<const x8*>(sm.Th + tpb[j] + rb * CK);
        tlf[b][j] = *reinterpret_cast<const x8*>(sm.Tl + tpb[j] + rb * CK);
      }
      fw4[b] = *reinterpret_cast<const float4*>(sm.F + 2 * CK + fb + rb);
    }

    // ---- Z = V - diag(fz) X as B operands (k = token) ----
    x8 Zh[NB][2], Zl[NB][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 z[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int b = 2 * j + hh;
          const float fzr[4] = {fz4[b].x, fz4[b].y, fz4[b].z, fz4[b].w};
#pragma unroll
          for (int r = 0; r < 4; ++r) z[hh][r] = M::dec(vraw[nb][b][r]) - fzr[r] * X[nb][b][r];
        }
        pack_split<TIN>(z[0], z[1], Zh[nb][j], Zl[nb][j]);
      }
    }

    // ---- U = T_b Z (lower triangular in token blocks) ----
    f32x4 U[NB][4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) U[nb][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j <= (b >> 1); ++j) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          U[nb][b] = M::mma(thf[b][j], Zh[nb][j], U[nb][b]);
          U[nb][b] = M::mma(thf[b][j], Zl[nb][j], U[nb][b]);
          U[nb][b] = M::mma(tlf[b][j], Zh[nb][j], U[nb][b]);
        }
      }
    }
    // P fragments and fo factors of O, read while U finishes
    x8 pff[4][2];
    float4 fo4[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int rb = 32 * (b >> 1) + 4 * (b & 1);
      if constexpr (OUTS) {
#pragma unroll
        for (int j = 0; j <= (b >> 1); ++j)
          pff[b][j] = *reinterpret_cast<const x8*>(sm.P + tpb[j] + rb * CK);
        fo4[b] = *reinterpret_cast<const float4*>(sm.F + CK + fb + rb);
      }
    }
    x8 Uh[NB][2], Ul[NB][2], Wh[NB][2], Wl[NB][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float4 fw[2] = {fw4[2 * j], fw4[2 * j + 1]};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const f32x4& u0 = U[nb][2 * j];
        const f32x4& u1 = U[nb][2 * j + 1];
        const f32x4 w0 = {fw[0].x * u0[0], fw[0].y * u0[1], fw[0].z * u0[2], fw[0].w * u0[3]};
        const f32x4 w1 = {fw[1].x * u1[0], fw[1].y * u1[1], fw[1].z * u1[2], fw[1].w * u1[3]};
        if constexpr (OUTS && kFullOut)
          pack_split<TIN>(u0, u1, Uh[nb][j], Ul[nb][j]);
        else if constexpr (OUTS)
          pack_hi<TIN>(u0, u1, Uh[nb][j]);
        pack_split<TIN>(w0, w1, Wh[nb][j], Wl[nb][j]);
      }
    }

    // ---- O = diag(fo) QS + P U, stored ----
#pragma unroll
    for (int b = 0; b < (OUTS ? 4 : 0); ++b) {
      const int rb = 32 * (b >> 1) + 4 * (b & 1);
      const float4 fo = fo4[b];
      f32x4 o[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        o[nb] = (f32x4){fo.x * QS[nb][b][0], fo.y * QS[nb][b][1], fo.z * QS[nb][b][2],
                        fo.w * QS[nb][b][3]};
#pragma unroll
      for (int j = 0; j <= (b >> 1); ++j) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          o[nb] = M::mma(pff[b][j], Uh[nb][j], o[nb]);
          if constexpr (kFullOut) {
            // P's low part, from the free quadrant of record part b / 2 + j
            const uint16_t* pq = (b >> 1) == 0 ? sm.Th : j == 0 ? sm.Tl : sm.P;
            const x8 pl = *reinterpret_cast<const x8*>(pq + tpb[1] + 4 * (b & 1) * CK);
            o[nb] = M::mma(pff[b][j], Ul[nb][j], o[nb]);
            o[nb] = M::mma(pl, Uh[nb][j], o[nb]);
          }
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (TOUT == kF32) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[nb][r]), orsrc,
                                                  lane_off + (rb + r) * out_row + 64 * nb +
                                                      blk_off[nb], 0, 0);
        } else {
          // 16-bit outputs go back through this wave's (already consumed) V
          // columns of the chunk buffer, to leave as whole 16-byte rows
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.V[vb[nb] + (rb + r) * VC] = OutT<TOUT>::enc(o[nb][r]);
        }
      }
    }

    // ---- St = e^{G_C} St + K^T W ----
    {
      // K^T fragments of key block kb + 1 are read while block kb multiplies
      auto read_kt = [&](x8 (&kd)[2], int kb) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint16_t* p = sm.K + trb[kb >> 1] + 32 * j * DKC + 4 * (kb & 1);
          const u16x4 t0 = lds_read_tr(p);
          const u16x4 t1 = lds_read_tr(p + 4 * DKC);
          const u16x8 kt = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
          kd[j] = __builtin_bit_cast(x8, kt);
        }
      };
      x8 ktf[2][2];
      read_kt(ktf[0], 0);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        if (kb < 7) read_kt(ktf[(kb + 1) & 1], kb + 1);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          f32x4 acc = St[nb][kb];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] *= gc;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            acc = M::mma(ktf[kb & 1][j], Wh[nb][j], acc);
            acc = M::mma(ktf[kb & 1][j], Wl[nb][j], acc);
          }
          St[nb][kb] = acc;
        }
      }
    }

    store_rows(cur, ch);
    lds_barrier();  // the chunk's buffer is free for the load wave
  };
  for (int ch = 0; ch < nch; ++ch) chunk_step(&sb[ch & 1], ch);

  store_state();
}

int64_t max_chunks(int64_t total_tokens, int64_t num_seqs) {
  return (total_tokens + CK - 1) / CK + num_seqs;
}

size_t meta_bytes(int64_t num_seqs) {
  return (size_t)((3 * num_seqs + 2 + kInfoWords) * 4 + 255) / 256 * 256;
}

// workgroups per walk of one v-head: enough for dv state rows, and for the Dk
// rows of a middle segment's transition walk
int walk_tiles(int dv) { return (std::max(dv, DKC) + WALK_BV - 1) / WALK_BV; }

// the split sequences' states (per split rank and v-head, each walk_tiles
// tiles of WALK_BV rows x Dk f32)
size_t seg_bytes(int64_t total_tokens, int64_t num_seqs, int hv, int dv) {
  const SegBounds b = seg_bounds(total_tokens, num_seqs);
  return (size_t)b.ranks * hv * b.slots() * walk_tiles(dv) * WALK_BV * DKC * sizeof(float);
}


constexpr int kMaxDevices = 64;

// The CU count of a device (asked once; racing first calls store the same value).
int device_cus(int dev) {
  static std::atomic<int> cus[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      return 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The fork and join events of the split schedule: two per host thread and
// device, created on the thread's first split call on that device and kept
// for the life of the process (a wait takes the event as it was recorded when
// the wait was enqueued, so later calls on the thread may record it again).
struct SplitEvents {
  hipEvent_t fork = nullptr, join = nullptr;
};
thread_local SplitEvents t_split_events[kMaxDevices];

const SplitEvents* split_events(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  SplitEvents& e = t_split_events[dev];
  if (!e.fork && hipEventCreateWithFlags(&e.fork, hipEventDisableTiming) != hipSuccess)
    e.fork = nullptr;
  if (!e.join && hipEventCreateWithFlags(&e.join, hipEventDisableTiming) != hipSuccess)
    e.join = nullptr;
  return e.fork && e.join ? &e : nullptr;
}

template <int TIN>
hipError_t launch_chunked_t(const PrefillArgs& a, void* ws, hipStream_t stream,
                            hipStream_t aux) {
  // workspace: metadata, the split sequences' states, the per-chunk records
  const MetaPtrs m = meta_ptrs(ws, a.num_seqs);
  float* segws = reinterpret_cast<float*>(static_cast<char*>(ws) + meta_bytes(a.num_seqs));
  char* recs = reinterpret_cast<char*>(segws) + seg_bytes(a.total_tokens, a.num_seqs, a.hv, a.dv);
  const int64_t mc = max_chunks(a.total_tokens, a.num_seqs);
  const int ntiles = walk_tiles(a.dv);
  const int per_seq_wgs = a.hv * ntiles;
  // the longest ranks may be split into segments (needs the ranking by length)
  const SegBounds sb = seg_bounds(a.total_tokens, a.num_seqs);
  const int ksmax = sb.ranks, smax = sb.smax;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  // The split schedule runs part of the call on the caller's second stream
  // `aux`, which must be on the caller's stream's device (the current one);
  // it is not used while the caller's stream is being captured.  The early
  // walk may take at most half of the CUs, so the records of the other ranks
  // always have room.
  bool can_split = aux != nullptr && aux != stream && a.num_seqs >= 2 &&
                   a.num_seqs <= kOrderMax;
  if (can_split) {
    hipDevice_t sdev = -1, adev = -1;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    can_split = hipStreamGetDevice(stream, &sdev) == hipSuccess && sdev == dev &&
                hipStreamGetDevice(aux, &adev) == hipSuccess && adev == dev &&
                hipStreamIsCapturing(stream, &cap) == hipSuccess &&
                cap == hipStreamCaptureStatusNone;
  }
  const int ncu = device_cus(dev);
  const SplitEvents* ev = can_split ? split_events(dev) : nullptr;
  int kmax = 0;
  if (ev)
    kmax = (int)std::min<int64_t>({(int64_t)kSplitMax, a.num_seqs - 1,
                                   (int64_t)(ncu / 2 / per_seq_wgs)});

  // In one stream order with few sequences the prep launch forms the
  // metadata itself (its workgroup 0); otherwise a launch of its own does.
  const bool self_meta = kmax == 0 && a.num_seqs <= kSelfMaxSeqs;
  const MetaIn mi{ntiles, ncu, ksmax, smax};
  if (!self_meta)
    hipLaunchKernelGGL(chunk_meta_kernel, dim3(1), dim3(256), 0, stream, a, m, ntiles, ncu, kmax,
                       ksmax, smax);

  const int64_t prep_units = mc * a.hk;
  if (prep_units + 1 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  auto prep = [&](int part, hipStream_t st) {
    if (part == kPartSelf)
      hipLaunchKernelGGL((chunk_prep_kernel<TIN, true>), dim3((unsigned)(prep_units + 1)),
                         dim3(256), 0, st, a, m, recs, part, mi);
    else
      hipLaunchKernelGGL((chunk_prep_kernel<TIN, false>), dim3((unsigned)prep_units), dim3(256),
                         0, st, a, m, recs, part, mi);
  };
  const int ratio = a.hv / a.hk;
  const size_t lds = 2 * sizeof(WalkBuf<WALK_NW, WALK_NB>);
  // walk items of a launch: at most one per rank, plus S - 1 more for each
  // split rank (phase B), or 2 S - 3 per split rank (phase A)
  auto walk_blocks = [&](int64_t items) {
    return (items * a.hk + kXcds - 1) / kXcds * kXcds * ratio * ntiles;
  };
  const int64_t seg_items = (int64_t)ksmax * (smax - 1);
  const int64_t a_items = (int64_t)ksmax * (2 * smax - 3);
  if (walk_blocks(a.num_seqs + seg_items) >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  // the dynamic-LDS limit is raised once per device and kernel: one mask per
  // kernel (outputs f32 / 16-bit, and the state-only walk)
  static std::atomic<uint64_t> raised_f32{0}, raised_16{0}, raised_st{0};
  auto walk = [&](int part, int64_t items, hipStream_t st, bool outs) -> hipError_t {
    auto go = [&](auto kern, std::atomic<uint64_t>& raised) -> hipError_t {
      const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
      if (!bit || !(raised.load(std::memory_order_acquire) & bit)) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
        raised.fetch_or(bit, std::memory_order_acq_rel);
      }
      hipLaunchKernelGGL(kern, dim3((unsigned)walk_blocks(items)), dim3(64 * (WALK_NW + 1)), lds, st,
                         a, m, (const char*)recs, segws, sb.slots(), ntiles, (int)mc, part);
      return hipSuccess;
    };
    if (!outs)
      return go(chunk_state_kernel<TIN, TIN, WALK_NW, WALK_NB, WALK_MINB, false>, raised_st);
    return a.out_dt == kF32
               ? go(chunk_state_kernel<TIN, kF32, WALK_NW, WALK_NB, WALK_MINB, true>, raised_f32)
               : go(chunk_state_kernel<TIN, TIN, WALK_NW, WALK_NB, WALK_MINB, true>, raised_16);
  };

  hipError_t e;
  if (kmax == 0) {
    // one stream: all records, the first phase of the split ranks (if the
    // device chose any), then every walk with outputs
    prep(self_meta ? kPartSelf : 2, stream);
    if (a_items > 0 && (e = walk(0, a_items, stream, false)) != hipSuccess) return e;
    if ((e = walk(2, a.num_seqs + seg_items, stream, true)) != hipSuccess) return e;
    return hipGetLastError();
  }
  // Split schedule (the rank k is chosen on the device; k = 0 leaves parts 0
  // empty and runs everything as part 1):
  //   caller's stream: meta, records of ranks [0, k), the first phase of the
  //                    split ranks among them, their walks
  //   aux stream:      (after those records) the other records, their walks
  // and the caller's stream then waits for the second.  The early walks are
  // queued right behind their records on the caller's stream, so they take
  // their CUs before the other records fill the device.
  prep(0, stream);
  if ((e = hipEventRecord(ev->fork, stream)) != hipSuccess) return e;
  if (a_items > 0 && (e = walk(0, a_items, stream, false)) != hipSuccess) return e;
  // the early part: at most kmax ranks, or all of them when there are few
  const int64_t early = a.num_seqs <= kSplitMax ? a.num_seqs : kmax;
  if ((e = walk(0, early + seg_items, stream, true)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(aux, ev->fork, 0)) != hipSuccess) return e;
  prep(1, aux);
  if ((e = walk(1, a.num_seqs, aux, true)) != hipSuccess) return e;
  if ((e = hipEventRecord(ev->join, aux)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(stream, ev->join, 0)) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace

bool chunked_supported(int in_dt, int out_dt, int64_t hv, int dk, int dv) {
  (void)out_dt;
  // the state walk addresses a chunk of output rows with 32-bit byte offsets
  const bool rows_fit = hv * dv * CK * (int64_t)sizeof(float) < ((int64_t)1 << 30);
  return (in_dt == kBF16 || in_dt == kF16) && dk == DKC && dv % 16 == 0 && dv >= 16 && rows_fit;
}

bool chunked_layout_ok(const void* q, const void* k, const void* v, int64_t q_rs, int64_t k_rs,
                       int64_t v_rs) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  // a chunk of rows is addressed with 32-bit byte offsets
  const int64_t lim = (int64_t)1 << 24;
  return al(q) && al(k) && al(v) && q_rs % 8 == 0 && k_rs % 8 == 0 && v_rs % 8 == 0 &&
         q_rs < lim && k_rs < lim && v_rs < lim;
}

size_t chunked_workspace_bytes(int64_t total_tokens, int64_t num_seqs, int hv, int dk, int dv) {
  (void)dk;
  return meta_bytes(num_seqs) + seg_bytes(total_tokens, num_seqs, hv, dv) +
         (size_t)max_chunks(total_tokens, num_seqs) * (size_t)hv * REC_BYTES;
}

hipError_t launch_prefill_chunked(const PrefillArgs& a, void* ws, size_t ws_bytes,
                                  hipStream_t stream, hipStream_t aux) {
  if (ws_bytes < chunked_workspace_bytes(a.total_tokens, a.num_seqs, a.hv, a.dk, a.dv))
    return hipErrorInvalidValue;
  if (a.num_seqs >= (1 << 30) || max_chunks(a.total_tokens, a.num_seqs) >= (1 << 30))
    return hipErrorInvalidValue;
  if (a.in_dt == kBF16) return launch_chunked_t<kBF16>(a, ws, stream, aux);
  if (a.in_dt == kF16) return launch_chunked_t<kF16>(a, ws, stream, aux);
  return hipErrorInvalidValue;
}

}  // namespace gdn
