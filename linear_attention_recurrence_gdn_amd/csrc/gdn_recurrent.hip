// gdn_recurrent.hip -- gate, single-token decode and token-sequential prefill
// kernels for gfx950.
//
// Method (vllm.cpp tests/vt/test_ops_gdn.cpp, "gdn decode: hand-computed
// single step"; Winery-Strata elementwise_parity.cpp, gdn_gate block):
//   g = softplus(alpha + dt_bias) * ssm_a  (softplus(x) = x when x > 20)
//   S *= exp(g);  v' = beta (v - S k);  S += v' k^T;  o = S (scale q)
// with q, k optionally L2-normalised (eps inside the square root) and v-head
// hv reading q/k head hv / (Hv / Hk).
//
// Decode is bound by HBM bandwidth: each (sequence, v-head) state is Dv x Dk
// fp32 (64 KiB at 128 x 128) that must be read and written once, against ~1
// flop per byte.  The layout of the work:
//   - one wavefront owns a tile of BV = NL * RPI state rows of one head; lane
//     l covers columns [4 (l % LPR), +4) of row r0 + i*RPI + l/LPR for
//     i < NL, with LPR = Dk/4 lanes per row and RPI = 64/LPR rows per load
//     instruction; every state access is a 16-byte load/store and each
//     instruction moves 1 KiB of contiguous state;
//   - all NL loads are issued before any arithmetic, so a wave keeps
//     16*NL bytes per lane in flight; NL = 8 (16 rows, 8 KiB of state per
//     wave at Dk = 128) and nontemporal loads/stores measured fastest: the
//     state is touched once per call, so it should not displace other lines
//     in the caches;
//   - S k and S q are reduced together from the OLD state with one
//     transposed butterfly, and the output uses
//       o = S_new q = decay (S_old q) + v' (k . q),
//     which is the same quantity, so the state is streamed exactly once;
//   - waves are independent: no LDS and no barriers.
#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_prefill_gate.h"

namespace gdn {

// ---------------------------------------------------------------------------
// gate
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gate_kernel(GateArgs a) {
  const int64_t n = a.rows * a.hv;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / a.hv;
    const int64_t h = i - r * a.hv;
    const float x = load1(a.alpha, a.alpha_dt, r * a.alpha_rs + h) + a.dt_bias[h];
    a.g[r * a.g_rs + h] = gate_value(x, a.ssm_a[h]);
    if (a.b) {
      const float bv = load1(a.b, a.alpha_dt, r * a.b_rs + h);
      const bool rnd = a.round_beta != 0;
      a.beta[r * a.beta_rs + h] = a.alpha_dt == kBF16 ? beta_from_raw<kBF16>(bv, rnd)
                                  : a.alpha_dt == kF16 ? beta_from_raw<kF16>(bv, rnd)
                                                       : beta_from_raw<kF32>(bv, rnd);
    }
  }
}

hipError_t launch_gate(const GateArgs& a, hipStream_t stream) {
  const int64_t n = a.rows * a.hv;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(gate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// shared per-token step on a wave's register tile
// ---------------------------------------------------------------------------
// The fused-norm decode runs one workgroup per (row, v-head) of at most this
// many waves (512 threads leave each lane up to 256 VGPRs: the doubled tile
// of the fused norm fits without spilling).
constexpr int kNormMaxWaves = 8;

template <int DK, int NL>
struct Tile {
  static constexpr int LPR = DK / 4;    // lanes per state row
  static constexpr int RPI = 64 / LPR;  // rows per load instruction
  static constexpr int BV = NL * RPI;   // rows per wave
  static_assert(NL <= LPR, "tile needs NL <= lanes per row");
  static constexpr int OWN = LPR / NL;  // lanes holding each reduced row
};

// q, k: this lane's 4 columns; returns normalised k in k4, scale*normalised q
// in q4 and (k . q) summed over the row.
template <int LPR>
__device__ __forceinline__ float prepare_qk(float4& q4, float4& k4, bool l2norm, float eps,
                                            float scale) {
  float qn = scale, kn = 1.0f;
  if (l2norm) {
    const float qq = group_sum<LPR>(dot4(q4, q4));
    const float kk = group_sum<LPR>(dot4(k4, k4));
    qn = scale / sqrtf(qq + eps);
    kn = 1.0f / sqrtf(kk + eps);
  }
  q4 = scale4(qn, q4);
  k4 = scale4(kn, k4);
  return group_sum<LPR>(dot4(k4, q4));
}

// One recurrence step on the wave's tile.  s[i] holds row r0 + i*RPI + sub.
// Returns, in every lane, the output of row `myrow` (see the caller).
template <int DK, int NL>
__device__ __forceinline__ float tile_step(float4 (&s)[NL], float4 q4, float4 k4, float kq,
                                           float decay, float beta, float vv, int lane,
                                           int sub) {
  using T = Tile<DK, NL>;
  float pk[NL], pq[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    pk[i] = dot4(s[i], k4);
    pq[i] = dot4(s[i], q4);
  }
  transpose_reduce<NL, T::LPR>(pk, lane);
  transpose_reduce<NL, T::LPR>(pq, lane);
  const float vp = beta * (vv - decay * pk[0]);
  const float o = decay * pq[0] + vp * kq;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const float vpi = __shfl(vp, sub * T::LPR + i * T::OWN, 64);
    s[i] = axpby4(decay, s[i], vpi, k4);
  }
  return o;
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------
// Wave -> (sequence b, v-head h, row tile) with the tile fastest, so the
// waves of one head are neighbours.  All indices are wave-uniform (scalar
// registers); the q/k/v/gate loads are issued before the slot index is
// waited on, and the whole state tile is requested before any arithmetic.
//
// NORM adds the gated RMSNorm after the step (vllm.cpp test_ops_gdn.cpp,
// "rmsnorm_gated: norm-then-gate"): the workgroup is then exactly the
// tiles_per_head waves of one (row, v-head), which add their squared outputs
// through LDS; each output is o / sqrt(mean(o^2) + eps) * w * act(z), from
// the unrounded f32 o.
template <int DK, int NL, int TIN, int TAL, int TS, bool NT, bool NORM>
__global__ __launch_bounds__(NORM ? 64 * kNormMaxWaves : 256) void decode_kernel(DecodeArgs a,
                                                                   int64_t total_waves,
                                                                   int tiles_per_head) {
  using T = Tile<DK, NL>;
  const int lane = threadIdx.x & 63;
  const uint32_t wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the host keeps the wave count below 2^31, so 32-bit index math suffices
  const uint32_t wave = blockIdx.x * (NORM ? (uint32_t)tiles_per_head : 4u) + wid;
  if (wave >= (uint32_t)total_waves) return;
  const int tile = (int)(wave % (uint32_t)tiles_per_head);
  const uint32_t bh = wave / (uint32_t)tiles_per_head;
  const int h = (int)(bh % (uint32_t)a.hv);
  const int64_t b = bh / (uint32_t)a.hv;
  const int r0 = tile * T::BV;
  const int sub = lane / T::LPR;
  const int col = (lane % T::LPR) * 4;
  const int j = (lane % T::LPR) / T::OWN;
  const int myrow = r0 + j * T::RPI + sub;
  const bool writer = (lane % T::OWN) == 0 && myrow < a.dv;
  const int64_t out_off = (b * a.hv + h) * a.dv + myrow;

  const int32_t slot = a.idx[b];
  const int hk = h / (a.hv / a.hk);
  const Raw4<TIN> qr = load_raw4<TIN>(a.q, b * a.q_rs + (int64_t)hk * DK + col, a.qk_vec != 0);
  const Raw4<TIN> kr = load_raw4<TIN>(a.k, b * a.k_rs + (int64_t)hk * DK + col, a.qk_vec != 0);
  const uint32_t vr = load_raw1<TIN>(a.v, b * a.v_rs + (int64_t)h * a.dv + min(myrow, a.dv - 1));
  const uint32_t ar = load_raw1<TAL>(a.alpha, b * a.alpha_rs + h);
  const float dtb = a.dt_bias[h];
  const float ssa = a.ssm_a[h];
  // beta is one value per (row, v-head): a wave-uniform scalar load either way
  const float beta =
      a.beta_raw ? beta_from_raw<TAL>(raw1_to_f32<TAL>(load_raw1<TAL>(a.beta, b * a.beta_rs + h)),
                                      true)
                 : static_cast<const float*>(a.beta)[b * a.beta_rs + h];
  uint32_t zr = 0, wr = 0;
  if constexpr (NORM) {
    const int row = min(myrow, a.dv - 1);
    zr = load_raw1<TIN>(a.norm_z, b * a.norm_z_rs + (int64_t)h * a.dv + row);
    wr = load_raw1<TIN>(a.norm_w, row);
  }

  // (block-uniform when NORM: every wave of the workgroup leaves here together)
  if (slot < 0 || slot >= a.num_slots) {
    // padded row: zeros; out-of-range slot (caller error): NaN.  No state access.
    if (writer) store1(a.out, a.out_dt, out_off, slot < 0 ? 0.0f : __builtin_nanf(""));
    return;
  }

  // element offset of this lane's columns in the (slot, head) state
  const int64_t S = (((int64_t)slot * a.hv + h) * a.dv) * DK + col;
  float4 s[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int row = min(r0 + i * T::RPI + sub, a.dv - 1);
    s[i] = state_load4<TS, NT>(a.pool, S + (int64_t)row * DK);
  }

  float4 q4 = raw_to_f32<TIN>(qr);
  float4 k4 = raw_to_f32<TIN>(kr);
  const float vv = raw1_to_f32<TIN>(vr);
  const float decay = expf(gate_value(raw1_to_f32<TAL>(ar) + dtb, ssa));
  const float kq = prepare_qk<T::LPR>(q4, k4, a.l2norm != 0, a.l2_eps, a.scale);
#pragma unroll
  for (int i = 0; i < NL; ++i)
    if (r0 + i * T::RPI + sub >= a.dv) s[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  float o = tile_step<DK, NL>(s, q4, k4, kq, decay, beta, vv, lane, sub);
  if constexpr (NORM) {
    __shared__ float part[kNormMaxWaves];
    const float sq = group_sum<64>(writer ? o * o : 0.0f);
    if (lane == 0) part[wid] = sq;
    __syncthreads();
    float tot = 0.0f;
    for (int i = 0; i < tiles_per_head; ++i) tot += part[i];
    const float inv = 1.0f / sqrtf(tot / (float)a.dv + a.norm_eps);
    o = o * inv * raw1_to_f32<TIN>(wr) * gate_act(raw1_to_f32<TIN>(zr), a.norm_sigmoid != 0);
  }
  if (writer) store1(a.out, a.out_dt, out_off, o);

#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int row = r0 + i * T::RPI + sub;
    if (row < a.dv) state_store4<TS, NT>(a.pool, S + (int64_t)row * DK, s[i]);
  }
}

template <int DK, int NL, int TIN, int TAL, int TS, bool NORM>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  using T = Tile<DK, NL>;
  const int tiles = (a.dv + T::BV - 1) / T::BV;
  const int64_t waves = a.batch * a.hv * tiles;
  if (waves >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if constexpr (NORM) {
    // one workgroup of `tiles` waves per (row, v-head)
    if (tiles > kNormMaxWaves) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_kernel<DK, NL, TIN, TAL, TS, true, true>),
                       dim3((unsigned)(a.batch * a.hv)), dim3(64 * tiles), 0, stream, a, waves,
                       tiles);
  } else {
    const int64_t blocks = (waves + 3) / 4;
    hipLaunchKernelGGL((decode_kernel<DK, NL, TIN, TAL, TS, true, false>),
                       dim3((unsigned)blocks), dim3(256), 0, stream, a, waves, tiles);
  }
  return hipGetLastError();
}

template <int DK, int NL, int TS, bool NORM>
static hipError_t launch_decode_ts(const DecodeArgs& a, hipStream_t stream) {
#define GDN_DEC(TI, TA) \
  if (a.in_dt == TI && a.alpha_dt == TA) return launch_decode_t<DK, NL, TI, TA, TS, NORM>(a, stream);
  GDN_DEC(kBF16, kF32) GDN_DEC(kF16, kF32) GDN_DEC(kF32, kF32)
  GDN_DEC(kBF16, kBF16) GDN_DEC(kF16, kBF16) GDN_DEC(kF32, kBF16)
  GDN_DEC(kBF16, kF16) GDN_DEC(kF16, kF16) GDN_DEC(kF32, kF16)
#undef GDN_DEC
  return hipErrorInvalidValue;
}

template <int DK, int NL, bool NORM>
static hipError_t launch_decode_st(const DecodeArgs& a, hipStream_t stream) {
  if (a.state_dt == kF32) return launch_decode_ts<DK, NL, kF32, NORM>(a, stream);
  if (a.state_dt == kBF16) return launch_decode_ts<DK, NL, kBF16, NORM>(a, stream);
  if (a.state_dt == kF16) return launch_decode_ts<DK, NL, kF16, NORM>(a, stream);
  return hipErrorInvalidValue;
}

// Loads per lane of the decode tile, per dk (measured fastest).  The fused
// norm doubles them where the row allows, so a head takes half the waves and
// a workgroup's barrier waits on fewer of them.
constexpr int decode_nl(int dk) { return dk == 16 ? 4 : 8; }
constexpr int decode_norm_nl(int dk) {
  return 2 * decode_nl(dk) <= dk / 4 ? 2 * decode_nl(dk) : decode_nl(dk);
}

template <int DK>
static hipError_t launch_decode_dk(const DecodeArgs& a, hipStream_t stream) {
  if (a.norm_z) return launch_decode_st<DK, decode_norm_nl(DK), true>(a, stream);
  return launch_decode_st<DK, decode_nl(DK), false>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  switch (a.dk) {
    case 16: return launch_decode_dk<16>(a, stream);
    case 32: return launch_decode_dk<32>(a, stream);
    case 64: return launch_decode_dk<64>(a, stream);
    case 128: return launch_decode_dk<128>(a, stream);
    case 256: return launch_decode_dk<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

// Largest dv the fused-norm decode takes for a given dk.
int decode_norm_max_dv(int dk) {
  switch (dk) {
    case 16: return kNormMaxWaves * Tile<16, decode_norm_nl(16)>::BV;
    case 32: return kNormMaxWaves * Tile<32, decode_norm_nl(32)>::BV;
    case 64: return kNormMaxWaves * Tile<64, decode_norm_nl(64)>::BV;
    case 128: return kNormMaxWaves * Tile<128, decode_norm_nl(128)>::BV;
    case 256: return kNormMaxWaves * Tile<256, decode_norm_nl(256)>::BV;
    default: return 0;
  }
}

// ---------------------------------------------------------------------------
// token-sequential prefill: one wave per (sequence, v-head, row tile) walks
// the sequence's tokens with its state tile in registers.  Token inputs are
// fetched PF tokens at a time into a register ring one group ahead of use,
// so each token's load latency is hidden behind the previous group's work.
// ---------------------------------------------------------------------------
template <int TIN>
struct TokenRaw {
  Raw4<TIN> q, k;
  uint32_t v;
  float g, beta;
};

template <int DK, int TIN>
__device__ __forceinline__ TokenRaw<TIN> load_token(const PrefillArgs& a, int64_t t, int hk,
                                                    int h, int col, int vrow) {
  TokenRaw<TIN> in;
  in.q = load_raw4<TIN>(a.q, t * a.q_rs + (int64_t)hk * DK + col, a.qk_vec != 0);
  in.k = load_raw4<TIN>(a.k, t * a.k_rs + (int64_t)hk * DK + col, a.qk_vec != 0);
  in.v = load_raw1<TIN>(a.v, t * a.v_rs + (int64_t)h * a.dv + vrow);
  token_gate(a, t, h, in.g, in.beta);
  return in;
}

template <int DK, int NL, int TIN, int PF>
__global__ __launch_bounds__(256) void prefill_seq_kernel(PrefillArgs a, int64_t total_waves,
                                                          int tiles_per_head) {
  using T = Tile<DK, NL>;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = blockIdx.x * 4u + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= (uint32_t)total_waves) return;
  const int tile = (int)(wave % (uint32_t)tiles_per_head);
  const uint32_t sh = wave / (uint32_t)tiles_per_head;
  const int h = (int)(sh % (uint32_t)a.hv);
  const int64_t sq = sh / (uint32_t)a.hv;
  const int r0 = tile * T::BV;
  const int sub = lane / T::LPR;
  const int col = (lane % T::LPR) * 4;
  const int j = (lane % T::LPR) / T::OWN;
  const int myrow = r0 + j * T::RPI + sub;
  const int vrow = min(myrow, a.dv - 1);
  const bool writer = (lane % T::OWN) == 0 && myrow < a.dv;

  // cu_seqlens is device data: clamp so a malformed table cannot index past
  // the token arrays.
  const int64_t t1 = min((int64_t)a.cu[sq + 1], a.total_tokens);
  const int64_t t0 = max((int64_t)0, min((int64_t)a.cu[sq], t1));
  const int64_t slot = a.idx ? (int64_t)a.idx[sq] : sq;
  if (slot < 0 || slot >= a.num_slots) {
    if (writer)
      for (int64_t t = t0; t < t1; ++t)
        store1(a.out, a.out_dt, (t * a.hv + h) * a.dv + myrow, __builtin_nanf(""));
    return;
  }
  const bool init = a.has_init ? a.has_init[sq] != 0 : true;
  const int hk = h / (a.hv / a.hk);
  const int64_t S = ((slot * a.hv + h) * a.dv) * DK + col;  // element offset in the pool

  if (t1 <= t0) {
    // a zero-length sequence reads no token row (with total_tokens == 0 the
    // token pointers may be null): its state passes through, or is zeroed
    // without an initial state
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int row = r0 + i * T::RPI + sub;
      if (row < a.dv)
        state_store4_rt(a.state_dt, a.pool, S + (int64_t)row * DK,
                        init ? state_load4_rt(a.state_dt, a.pool, S + (int64_t)row * DK)
                             : make_float4(0.f, 0.f, 0.f, 0.f));
    }
    return;
  }

  // token rows t0 .. t1 - 1 exist from here on
  TokenRaw<TIN> cur[PF], nxt[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u)
    cur[u] = load_token<DK, TIN>(a, min(t0 + u, t1 - 1), hk, h, col, vrow);

  float4 s[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int row = min(r0 + i * T::RPI + sub, a.dv - 1);
    s[i] = init ? state_load4_rt(a.state_dt, a.pool, S + (int64_t)row * DK)
                : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < NL; ++i)
    if (r0 + i * T::RPI + sub >= a.dv) s[i] = make_float4(0.f, 0.f, 0.f, 0.f);

  for (int64_t base = t0; base < t1; base += PF) {
    // next group: clamped to the last token (a re-read, never out of range)
#pragma unroll
    for (int u = 0; u < PF; ++u)
      nxt[u] = load_token<DK, TIN>(a, min(base + PF + u, t1 - 1), hk, h, col, vrow);
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int64_t t = base + u;
      if (t < t1) {
        float4 q4 = raw_to_f32<TIN>(cur[u].q);
        float4 k4 = raw_to_f32<TIN>(cur[u].k);
        const float kq = prepare_qk<T::LPR>(q4, k4, a.l2norm != 0, a.l2_eps, a.scale);
        const float o = tile_step<DK, NL>(s, q4, k4, kq, expf(cur[u].g), cur[u].beta,
                                          raw1_to_f32<TIN>(cur[u].v), lane, sub);
        if (writer) store1(a.out, a.out_dt, (t * a.hv + h) * a.dv + myrow, o);
      }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u) cur[u] = nxt[u];
  }
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int row = r0 + i * T::RPI + sub;
    if (row < a.dv) state_store4_rt(a.state_dt, a.pool, S + (int64_t)row * DK, s[i]);
  }
}

template <int DK, int NL, int TIN>
static hipError_t launch_prefill_seq_t(const PrefillArgs& a, hipStream_t stream) {
  using T = Tile<DK, NL>;
  constexpr int PF = 8;
  const int tiles = (a.dv + T::BV - 1) / T::BV;
  const int64_t waves = a.num_seqs * a.hv * tiles;
  if (waves >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((prefill_seq_kernel<DK, NL, TIN, PF>), dim3((unsigned)blocks), dim3(256), 0,
                     stream, a, waves, tiles);
  return hipGetLastError();
}

template <int DK, int NL>
static hipError_t launch_prefill_seq_dk(const PrefillArgs& a, hipStream_t stream) {
  if (a.in_dt == kBF16) return launch_prefill_seq_t<DK, NL, kBF16>(a, stream);
  if (a.in_dt == kF16) return launch_prefill_seq_t<DK, NL, kF16>(a, stream);
  if (a.in_dt == kF32) return launch_prefill_seq_t<DK, NL, kF32>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_sequential(const PrefillArgs& a, hipStream_t stream) {
  switch (a.dk) {
    case 16: return launch_prefill_seq_dk<16, 1>(a, stream);
    case 32: return launch_prefill_seq_dk<32, 2>(a, stream);
    case 64: return launch_prefill_seq_dk<64, 4>(a, stream);
    case 128: return launch_prefill_seq_dk<128, 4>(a, stream);
    case 256: return launch_prefill_seq_dk<256, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
