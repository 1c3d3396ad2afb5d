"""Seeded synthetic inputs for the Gated DeltaNet hot path.

This module is shared by the GPU library's tests/bench and by the CPU oracle's
tests.  It only draws random numbers and encodes them into the byte layouts the
two sides read (f32, IEEE binary16, bfloat16); it contains none of the method's
arithmetic (no gate, no normalisation, no recurrence).  ``ssm_a = -exp(A_log)``
and ``beta = sigmoid(b)`` are input preparations that happen before the hot
path (the gate consumes ``ssm_a`` and the recurrence consumes the
post-sigmoid ``beta``), so they are done here once, in f64, and rounded to f32.

Value regimes follow the pages' workloads: L2-normalised-later q/k drawn from
N(0,1), negative log-decays from ``ssm_a < 0``, beta in (0,1), a large-alpha
head that crosses the softplus branch (Winery-Strata ``elementwise_parity.cpp``,
the ``gdn_gate`` fixture), and Dk=Dv=128 heads with GQA (vllm.cpp
``test_ops_gdn.cpp``, the packed decode and chunked prefill cases).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2}


# --------------------------------------------------------------------------
# encodings (storage formats only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round f32 values to bfloat16 bit patterns, nearest-even; a NaN keeps its
    top 16 bits with the quiet bit forced (the rule Winery-Strata's
    ``f32_to_bf16_bulk`` check states)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    b = x32.view(np.uint32).astype(np.uint64)
    rounded = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    quiet = ((b >> 16) | 0x40).astype(np.uint16)
    return np.where(np.isnan(x32), quiet, rounded)


def encode(x, dtype: int) -> np.ndarray:
    """f64/f32 values -> storage array (float32, float16, or uint16 bf16 bits)."""
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        return np.ascontiguousarray(np.asarray(x, dtype=np.float32).astype(np.float16))
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype}")


def decode_to_f32(a: np.ndarray, dtype: int) -> np.ndarray:
    """Storage array -> float32 view of the same values (for reporting only)."""
    if dtype == F32:
        return a.astype(np.float32)
    if dtype == F16:
        return a.astype(np.float32)
    if dtype == BF16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(f"unknown dtype {dtype}")


F16_NAN_BITS = 0x7E00      # canary written into padding columns
BF16_NAN_BITS = 0x7FC0


def nan_fill(shape, dtype: int) -> np.ndarray:
    if dtype == F32:
        return np.full(shape, np.nan, dtype=np.float32)
    if dtype == F16:
        return np.full(shape, F16_NAN_BITS, dtype=np.uint16).view(np.float16)
    return np.full(shape, BF16_NAN_BITS, dtype=np.uint16)


# --------------------------------------------------------------------------
# state pools: counter-based per-slot streams, so any slot can be regenerated
# on its own (the full-size cases sample slots without materialising twice)
# --------------------------------------------------------------------------
def pool_slot(seed: int, slot: int, hv: int, dv: int, dk: int, std: float) -> np.ndarray:
    rng = np.random.default_rng([seed, 0x5107, slot])
    s = rng.standard_normal(hv * dv * dk, dtype=np.float32)
    s *= np.float32(std)
    return s.reshape(hv, dv, dk)


def make_pool(seed: int, slots: int, hv: int, dv: int, dk: int, std: float) -> np.ndarray:
    pool = np.empty((slots, hv, dv, dk), dtype=np.float32)
    for s in range(slots):
        pool[s] = pool_slot(seed, s, hv, dv, dk, std)
    return pool


# --------------------------------------------------------------------------
# gate-side inputs
# --------------------------------------------------------------------------
def gate_inputs(rng, rows: int, hv: int, *, large_every_third: bool,
                head0_offset: float, a_log_hi: float):
    """alpha [rows,hv] f32, dt_bias [hv] f32, ssm_a [hv] f32 (= -exp(A_log))."""
    alpha = rng.normal(0.0, 3.0, size=(rows, hv))
    if large_every_third:
        big = rng.uniform(22.0, 120.0, size=(rows, hv))
        heads = (np.arange(hv) % 3) == 0
        alpha[:, heads] = big[:, heads]
    if head0_offset:
        alpha[:, 0] += head0_offset
    dt_bias = rng.normal(0.0, 0.5, size=hv)
    a_log = rng.uniform(0.0, a_log_hi, size=hv)
    ssm_a = -np.exp(a_log)
    return (alpha.astype(np.float32), dt_bias.astype(np.float32),
            ssm_a.astype(np.float32))


def beta_inputs(rng, rows: int, hv: int) -> np.ndarray:
    b = rng.normal(0.0, 1.0, size=(rows, hv))
    return (1.0 / (1.0 + np.exp(-b))).astype(np.float32)


# --------------------------------------------------------------------------
# cases
# --------------------------------------------------------------------------
@dataclass
class View:
    """A [rows, heads, dim] operand inside a (possibly shared) 2-D buffer:
    element (r, h, d) is at ``buf.flat[r*row_stride + offset + h*dim + d]``."""
    buf: np.ndarray
    offset: int
    row_stride: int
    dtype: int


@dataclass
class DecodeCase:
    name: str
    batch: int
    hk: int
    hv: int
    dk: int
    dv: int
    in_dtype: int
    out_dtype: int
    q: View
    k: View
    v: View
    alpha: np.ndarray          # [B, hv] f32 (row stride hv)
    dt_bias: np.ndarray        # [hv] f32
    ssm_a: np.ndarray          # [hv] f32, negative
    beta: np.ndarray           # [B, hv] f32
    pool: np.ndarray           # [slots, hv, dv, dk] f32
    idx: np.ndarray            # [B] int32, -1 = padded row
    scale: float
    l2_eps: float = 1e-6
    l2norm: bool = True
    pool_seed: Optional[int] = None
    pool_std: float = 0.0
    meta: dict = field(default_factory=dict)

    @property
    def num_slots(self) -> int:
        return self.pool.shape[0]


@dataclass
class PrefillCase:
    name: str
    total_tokens: int
    num_seqs: int
    hk: int
    hv: int
    dk: int
    dv: int
    in_dtype: int
    out_dtype: int
    q: View
    k: View
    v: View
    alpha: np.ndarray          # [T, hv] f32
    dt_bias: np.ndarray
    ssm_a: np.ndarray
    beta: np.ndarray           # [T, hv] f32
    cu_seqlens: np.ndarray     # [N+1] int32
    pool: np.ndarray           # [slots, hv, dv, dk] f32
    idx: np.ndarray            # [N] int32
    has_init: np.ndarray       # [N] int8
    scale: float
    l2_eps: float = 1e-6
    l2norm: bool = True
    meta: dict = field(default_factory=dict)

    @property
    def num_slots(self) -> int:
        return self.pool.shape[0]


def _contig_view(x: np.ndarray, dtype: int) -> View:
    rows = x.shape[0]
    flat = np.ascontiguousarray(x).reshape(rows, -1)
    return View(flat, 0, flat.shape[1], dtype)


def make_decode_case(name: str, seed: int, *, batch: int, hk: int, hv: int, dk: int,
                     dv: int, in_dtype: int, out_dtype: int, slots: int,
                     pool_std: float = 0.05, large_every_third: bool = False,
                     head0_offset: float = 40.0, a_log_hi: float = 2.0,
                     packed_pad: Optional[int] = None, null_rows=(),
                     scale: Optional[float] = None, with_pool: bool = True) -> DecodeCase:
    """One decode step for `batch` single-token sequences whose states live in a
    `slots`-slot pool.  idx = prefix of a seeded permutation of the slots, with
    the rows listed in `null_rows` set to -1.  With `packed_pad`, q|k|v share
    one row of width 2*hk*dk + hv*dv + packed_pad (padding = NaN canaries).
    `with_pool=False` leaves `pool` as an empty [0, hv, dv, dk] array, for a
    caller that fills the slots itself (timing only)."""
    assert slots >= batch
    rng = np.random.default_rng(seed)
    q = rng.normal(0.0, 1.0, size=(batch, hk, dk))
    k = rng.normal(0.0, 1.0, size=(batch, hk, dk))
    v = rng.normal(0.0, 1.0, size=(batch, hv, dv))
    alpha, dt_bias, ssm_a = gate_inputs(rng, batch, hv, large_every_third=large_every_third,
                                        head0_offset=head0_offset, a_log_hi=a_log_hi)
    beta = beta_inputs(rng, batch, hv)
    perm = rng.permutation(slots).astype(np.int32)
    idx = perm[:batch].copy()
    for r in null_rows:
        idx[r] = -1
    if packed_pad is None:
        qv, kv, vv = (_contig_view(encode(q, in_dtype), in_dtype),
                      _contig_view(encode(k, in_dtype), in_dtype),
                      _contig_view(encode(v, in_dtype), in_dtype))
    else:
        width = 2 * hk * dk + hv * dv
        stride = width + packed_pad
        buf = nan_fill((batch, stride), in_dtype)
        buf[:, 0:hk * dk] = encode(q.reshape(batch, -1), in_dtype)
        buf[:, hk * dk:2 * hk * dk] = encode(k.reshape(batch, -1), in_dtype)
        buf[:, 2 * hk * dk:width] = encode(v.reshape(batch, -1), in_dtype)
        qv = View(buf, 0, stride, in_dtype)
        kv = View(buf, hk * dk, stride, in_dtype)
        vv = View(buf, 2 * hk * dk, stride, in_dtype)
    pool = (make_pool(seed, slots, hv, dv, dk, pool_std) if with_pool
            else np.empty((0, hv, dv, dk), np.float32))
    return DecodeCase(name=name, batch=batch, hk=hk, hv=hv, dk=dk, dv=dv,
                      in_dtype=in_dtype, out_dtype=out_dtype, q=qv, k=kv, v=vv,
                      alpha=alpha, dt_bias=dt_bias, ssm_a=ssm_a, beta=beta, pool=pool,
                      idx=idx, scale=float(np.float32(1.0 / np.sqrt(dk)) if scale is None
                                            else np.float32(scale)),
                      pool_seed=seed, pool_std=pool_std)


def make_prefill_case(name: str, seed: int, *, lengths, hk: int, hv: int, dk: int, dv: int,
                      in_dtype: int, out_dtype: int, slots: int, pool_std: float = 0.05,
                      has_init=None, head0_offset: float = 40.0, a_log_hi: float = 2.0,
                      nan_uninit_slots: bool = True, scale: Optional[float] = None,
                      ) -> PrefillCase:
    """Varlen prefill over sequences of the given lengths packed back to back.
    Sequence s starts from pool[idx[s]] when has_init[s] (else from zeros; the
    slot is then filled with NaN, which must never be read) and its final
    state is written back to pool[idx[s]]."""
    lengths = [int(x) for x in lengths]
    n = len(lengths)
    assert slots >= n
    t = int(sum(lengths))
    rng = np.random.default_rng(seed)
    q = rng.normal(0.0, 1.0, size=(t, hk, dk))
    k = rng.normal(0.0, 1.0, size=(t, hk, dk))
    v = rng.normal(0.0, 1.0, size=(t, hv, dv))
    alpha, dt_bias, ssm_a = gate_inputs(rng, t, hv, large_every_third=False,
                                        head0_offset=head0_offset, a_log_hi=a_log_hi)
    beta = beta_inputs(rng, t, hv)
    perm = rng.permutation(slots).astype(np.int32)
    idx = perm[:n].copy()
    if has_init is None:
        has_init = np.ones(n, dtype=np.int8)
    has_init = np.asarray(has_init, dtype=np.int8)
    cu = np.zeros(n + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    pool = make_pool(seed, slots, hv, dv, dk, pool_std)
    if nan_uninit_slots:
        for s in range(n):
            if not has_init[s]:
                pool[idx[s]] = np.nan
    return PrefillCase(name=name, total_tokens=t, num_seqs=n, hk=hk, hv=hv, dk=dk, dv=dv,
                       in_dtype=in_dtype, out_dtype=out_dtype,
                       q=_contig_view(encode(q, in_dtype), in_dtype),
                       k=_contig_view(encode(k, in_dtype), in_dtype),
                       v=_contig_view(encode(v, in_dtype), in_dtype),
                       alpha=alpha, dt_bias=dt_bias, ssm_a=ssm_a, beta=beta,
                       cu_seqlens=cu, pool=pool, idx=idx, has_init=has_init,
                       scale=float(np.float32(1.0 / np.sqrt(dk)) if scale is None
                                   else np.float32(scale)),
                       meta={"lengths": lengths})


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------
def tiny_prefill_then_decode(seed: int = 101):
    """T=64 f32 prefill of one sequence (Hk=Hv=2, Dk=Dv=16, scale 1/4) from a
    N(0, 0.1^2) state, then 4 decode steps (B=1, idx=[0]) with fresh draws."""
    pre = make_prefill_case("tiny-prefill-T64-f32", seed, lengths=[64], hk=2, hv=2, dk=16,
                            dv=16, in_dtype=F32, out_dtype=F32, slots=1, pool_std=0.1)
    steps = [make_decode_case(f"tiny-decode-step{i}", seed * 100 + i, batch=1, hk=2, hv=2,
                              dk=16, dv=16, in_dtype=F32, out_dtype=F32, slots=1)
             for i in range(4)]
    return pre, steps


def decode_b256(seed: int = 202) -> DecodeCase:
    """B=256 single-token decode, Hk=16, Hv=32 (GQA 2), D=128, bf16 q/k/v/out,
    fp32 pool of 1024 slots, every third head's alpha U(22,120), A_log U(0,2.8)."""
    return make_decode_case("decode-B256-Hk16-Hv32-D128-bf16", seed, batch=256, hk=16, hv=32,
                            dk=128, dv=128, in_dtype=BF16, out_dtype=BF16, slots=1024,
                            pool_std=0.05, large_every_third=True, head0_offset=0.0,
                            a_log_hi=2.8)


def prefill_t4096(seed: int = 303) -> PrefillCase:
    """One sequence T=4096, Hk=16, Hv=32, D=128, bf16, zero initial state."""
    return make_prefill_case("prefill-T4096-Hk16-Hv32-D128-bf16", seed, lengths=[4096],
                             hk=16, hv=32, dk=128, dv=128, in_dtype=BF16, out_dtype=BF16,
                             slots=1, has_init=[0])


def varlen_lengths(seed: int = 404, n: int = 8, total: int = 32768, hi: int = 8192):
    rng = np.random.default_rng([seed, 0x1E4])
    while True:
        head = rng.integers(1, hi + 1, size=n - 1)
        last = total - int(head.sum())
        if 1 <= last <= hi:
            return [int(x) for x in head] + [last]


def prefill_varlen_gqa3(seed: int = 404) -> PrefillCase:
    """8 sequences, lengths U(1,8192) summing to 32768, Hk=8, Hv=24 (GQA 3), D=128,
    fp16, initial states gathered from a 64-slot pool by index."""
    return make_prefill_case("prefill-varlen8-T32768-Hk8-Hv24-D128-f16", seed,
                             lengths=varlen_lengths(seed), hk=8, hv=24, dk=128, dv=128,
                             in_dtype=F16, out_dtype=F16, slots=64, pool_std=0.05)


def decode_packed_b1024(seed: int = 505, with_pool: bool = True) -> DecodeCase:
    """B=1024 decode from one packed fp16 q|k|v row per sequence (stride padded by
    256 NaN columns), Hk=16, Hv=32, D=128, fp32 pool of 4096 slots."""
    return make_decode_case("decode-packed-B1024-Hk16-Hv32-D128-f16", seed, batch=1024,
                            hk=16, hv=32, dk=128, dv=128, in_dtype=F16, out_dtype=F16,
                            slots=4096, pool_std=0.05, packed_pad=256, with_pool=with_pool)


# --------------------------------------------------------------------------
# gated RMSNorm inputs (the norm after the recurrence)
# --------------------------------------------------------------------------
@dataclass
class NormInputs:
    z: View                  # gate [rows, hv, dv] inside padded token rows
    w: np.ndarray            # [dv] weight, storage dtype
    dtype: int
    eps: float = 1e-6


def norm_inputs(seed: int, rows: int, hv: int, dv: int, dtype: int, *, pad: int = 0,
                z_range: float = 6.0) -> NormInputs:
    """Gate z ~ U(-z_range, z_range) in token rows of hv*dv + pad elements (the
    padding holds NaN, which must never be read) and weight w ~ U(-1, 1),
    encoded in `dtype` (the ranges of the pages' gated-norm kernel tests)."""
    rng = np.random.default_rng([seed, 0x9A7E])
    z = rng.uniform(-z_range, z_range, size=(rows, hv * dv))
    w = rng.uniform(-1.0, 1.0, size=dv)
    buf = nan_fill((rows, hv * dv + pad), dtype)
    buf[:, :hv * dv] = encode(z, dtype)
    return NormInputs(z=View(np.ascontiguousarray(buf), 0, hv * dv + pad, dtype),
                      w=encode(w, dtype), dtype=dtype)


# --------------------------------------------------------------------------
# merged b|a projection rows (the packed in_proj_ba layout)
# --------------------------------------------------------------------------
@dataclass
class MergedBA:
    buf: np.ndarray          # [rows, prefix + 2*hv + suffix] storage, NaN canaries around
    b_off: int               # column of b[., 0]
    a_off: int               # column of a[., 0]
    row_stride: int
    dtype: int


def merged_ba(seed: int, alpha: np.ndarray, dtype: int, *, prefix: int = 1, suffix: int = 3,
              b_range: float = 3.0) -> MergedBA:
    """Rows holding b in columns [prefix, prefix+hv) and a (= alpha, the raw
    gate projection) in [prefix+hv, prefix+2hv), NaN elsewhere; raw b ~
    U(-b_range, b_range), all encoded in `dtype`."""
    rows, hv = alpha.shape
    rng = np.random.default_rng([seed, 0xBA])
    b = rng.uniform(-b_range, b_range, size=(rows, hv))
    width = prefix + 2 * hv + suffix
    buf = nan_fill((rows, width), dtype)
    buf[:, prefix:prefix + hv] = encode(b, dtype)
    buf[:, prefix + hv:prefix + 2 * hv] = encode(alpha, dtype)
    return MergedBA(buf=np.ascontiguousarray(buf), b_off=prefix, a_off=prefix + hv,
                    row_stride=width, dtype=dtype)
