"""Helpers that run the seeded workload cases through the HIP library and
compare them with the oracle's f64 results.  Used by the GPU tests, smoke()
and bench.py's parity spot check."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

import workloads as W
import linear_attention_recurrence_gdn_amd as gdn

TORCH_OF = {W.F32: torch.float32, W.F16: torch.float16, W.BF16: torch.bfloat16}

# Bars.  Relative L1 = sum|got - want| / sum|want|, accumulated in f64, both
# over the whole tensor and over every unit on its own ((row or token, v-head)
# for outputs, (row or sequence, v-head) for states), so one wrong unit cannot
# hide in a large tensor:
OUT_TOL_F32 = 1e-5       # outputs, f32 inputs and outputs
OUT_TOL_HALF_F32 = 2e-3  # outputs, bf16 / fp16 inputs and f32 outputs
OUT_TOL_HALF = 2e-2      # outputs stored as bf16 / fp16
STATE_TOL = 1e-4         # fp32 states
# Elementwise, |got - want| <= atol + rtol |want| for every element (vllm.cpp
# test_ops_gdn.cpp CheckClose with its CUDA dtype combos: f32 -> f32,
# bf16 -> f32, bf16 -> bf16; fp16 takes the bf16 entries).
CLOSE_F32 = (1e-5, 1e-5)
CLOSE_HALF_F32 = (2e-3, 2e-3)
CLOSE_HALF = (4e-3, 8e-3)


def rel_l1(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    d = np.abs(got - want).sum()
    m = np.abs(want).sum()
    return float(d / max(m, 1e-30))


# A unit's relative L1 is taken against max(its own L1, UNIT_FLOOR x the mean
# unit's L1): an absolute floor, as the atol of an elementwise bar.  A unit
# far smaller than its neighbours (an output row whose k.q nearly cancels)
# carries the rounding error of the large terms that cancelled, which is not
# small relative to the unit itself; a unit that is wrong outright still
# scores at least UNIT_FLOOR, above every bar.
UNIT_FLOOR = 0.1


def unit_rel_l1(got, want, unit_dims: int) -> np.ndarray:
    """Relative L1 of every unit: the leading `unit_dims` axes index the units,
    the rest are summed."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    axes = tuple(range(unit_dims, got.ndim))
    d = np.abs(got - want).sum(axis=axes)
    m = np.abs(want).sum(axis=axes)
    floor = UNIT_FLOOR * float(m.mean()) if m.size else 0.0
    return d / np.maximum(np.maximum(m, floor), 1e-30)


def tier_tol(in_dtype, out_dtype) -> float:
    """The relative-L1 bar of an output: f32 in and out, 16-bit in with f32
    out, or a 16-bit stored output."""
    if in_dtype == W.F32 and out_dtype == W.F32:
        return OUT_TOL_F32
    return OUT_TOL_HALF_F32 if out_dtype == W.F32 else OUT_TOL_HALF


def out_tol(case) -> float:
    return tier_tol(case.in_dtype, case.out_dtype)


def close_tol(in_dtype, out_dtype):
    if in_dtype == W.F32:
        return CLOSE_F32
    return CLOSE_HALF_F32 if out_dtype == W.F32 else CLOSE_HALF


def diff_stats(got, want):
    """(max |got - want|, mean |got - want|)."""
    d = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))
    return (float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0)


def check_close(got, want, atol: float, rtol: float, name: str):
    """Every element within atol + rtol |want| (NaN fails)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    ok = np.abs(got - want) <= atol + rtol * np.abs(want)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} elements outside {atol:g} + {rtol:g}|want|; "
                             f"first at {i}: got {got[i]!r} want {want[i]!r}")


def check_units(got, want, unit_dims: int, tol: float, name: str) -> float:
    """Pooled and per-unit relative L1 within tol; returns the worst unit's."""
    r = rel_l1(got, want)
    assert r <= tol, f"{name}: rel-L1 {r:.3e} > {tol:g}"
    u = unit_rel_l1(got, want, unit_dims)
    if u.size:
        worst = np.unravel_index(int(np.argmax(u)), u.shape)
        assert u[worst] <= tol, f"{name}: unit {worst} rel-L1 {u[worst]:.3e} > {tol:g}"
        return float(u[worst])
    return 0.0


def to_dev(buf: np.ndarray, dtype: int, dev) -> torch.Tensor:
    """Storage array -> device tensor of the storage dtype (same bytes)."""
    if dtype == W.BF16:
        t = torch.from_numpy(np.ascontiguousarray(buf).view(np.int16)).to(dev)
        return t.view(torch.bfloat16)
    if dtype == W.F16:
        return torch.from_numpy(np.ascontiguousarray(buf).view(np.float16)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(buf, dtype=np.float32)).to(dev)


def view_of(dbufs: dict, v: W.View, rows: int, heads: int, dim: int) -> torch.Tensor:
    t = dbufs[id(v.buf)]
    flat = t.reshape(-1)
    return flat.as_strided((rows, heads, dim), (v.row_stride, dim, 1), v.offset)


def upload_views(case, dev, rows):
    dbufs = {}
    for v in (case.q, case.k, case.v):
        if id(v.buf) not in dbufs:
            dbufs[id(v.buf)] = to_dev(v.buf, v.dtype, dev)
    q = view_of(dbufs, case.q, rows, case.hk, case.dk)
    k = view_of(dbufs, case.k, rows, case.hk, case.dk)
    v = view_of(dbufs, case.v, rows, case.hv, case.dv)
    return dbufs, q, k, v


def bytes_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Byte-wise equality (NaN canaries compare equal to themselves)."""
    return torch.equal(a.contiguous().view(-1).view(torch.uint8),
                       b.contiguous().view(-1).view(torch.uint8))


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


# ---- 16-bit state pools ----------------------------------------------------
STATE_MANT_BITS = {W.F16: 10, W.BF16: 7}
STATE_MIN_EXP = {W.F16: -14, W.BF16: -126}


def pool_storage(pool_f32: np.ndarray, state_dt: int) -> np.ndarray:
    """The pool as stored: the f32 array itself, or the uint16 bits of its
    round-to-nearest-even f16 / bf16 encoding."""
    if state_dt == W.F32:
        return pool_f32
    return np.ascontiguousarray(W.encode(pool_f32, state_dt)).view(np.uint16)


def check_state_rounded(got: np.ndarray, want: np.ndarray, state_dt: int, name: str) -> float:
    """A 16-bit stored state against the oracle's f64 state: each element is
    within half a unit in the last place of its binade (the one rounding on
    store) plus an allowance for the f32 arithmetic before it (the f32-state
    tolerance, 1e-4, against the mean magnitude); and at least 90 % of the
    elements are the nearest 16-bit value to the oracle's (a truncating or
    otherwise wrong rounding misses about half of them)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    mag = np.abs(want)
    e = np.floor(np.log2(np.maximum(mag, 2.0 ** STATE_MIN_EXP[state_dt])))
    half_ulp = np.ldexp(0.5, (e - STATE_MANT_BITS[state_dt]).astype(np.int64))
    allow = half_ulp + 2e-5 * mag + STATE_TOL * float(mag.mean())
    err = np.abs(got - want)
    bad = ~(err <= allow)
    assert not bad.any(), (f"{name}: {int(bad.sum())} state elements off by more than half "
                           f"an ulp (worst {float((err / allow).max()):.2f} x allowance)")
    nearest = pool_storage(want.astype(np.float32), state_dt)
    nearest = nearest.view(np.float16) if state_dt == W.F16 else nearest
    hit = float(np.mean(W.decode_to_f32(nearest, state_dt).astype(np.float64) == got))
    assert hit >= 0.9, f"{name}: only {hit:.1%} of the state elements are the nearest value"
    r = rel_l1(got, want)
    assert r <= 2.0 ** -(STATE_MANT_BITS[state_dt] + 1), f"{name}: state rel-L1 {r:.3e}"
    return r


def _state_dt_of(pool: torch.Tensor) -> int:
    return {torch.float32: W.F32, torch.float16: W.F16, torch.bfloat16: W.BF16}[pool.dtype]


def _check_state(got: torch.Tensor, want: np.ndarray, name: str, tol: float,
                 in_dtype: int = W.F32) -> float:
    """A state tensor [units..., dv, dk] against the oracle's f64 states: f32
    storage by pooled and per-(row or sequence, v-head) relative L1 plus the
    elementwise bar of the input dtype's combo; 16-bit storage by the rounding
    checker (every element)."""
    sdt = _state_dt_of(got)
    got64 = got.float().cpu().numpy()
    if sdt == W.F32:
        check_units(got64, want, got64.ndim - 2, tol, f"{name} state")
        check_close(got64, want, *close_tol(in_dtype, W.F32), f"{name} state")
        return rel_l1(got64, want)
    return check_state_rounded(got64, want, sdt, name)


@dataclass
class DecodeResult:
    out: np.ndarray            # [B, hv, dv] f64 (values the GPU stored)
    pool: torch.Tensor         # device pool after the call
    pool0: Optional[torch.Tensor]  # device copy of the pool before the call
    inputs_unchanged: bool


def run_decode(case: W.DecodeCase, dev, *, keep_pool0: bool = True, pool=None,
               out_dtype=None) -> DecodeResult:
    dbufs, q, k, v = upload_views(case, dev, case.batch)
    snap = [t.clone() for t in dbufs.values()]
    alpha = torch.from_numpy(case.alpha).to(dev)
    dt_bias = torch.from_numpy(case.dt_bias).to(dev)
    ssm_a = torch.from_numpy(case.ssm_a).to(dev)
    beta = torch.from_numpy(case.beta).to(dev)
    idx = torch.from_numpy(case.idx).to(dev)
    if pool is None:
        pool = torch.from_numpy(case.pool).to(dev)
    pool0 = pool.clone() if keep_pool0 else None
    out = gdn.decode(q, k, v, alpha, dt_bias, ssm_a, beta, pool, idx, scale=case.scale,
                     l2norm=case.l2norm, l2_eps=case.l2_eps,
                     out_dtype=out_dtype or TORCH_OF[case.out_dtype])
    torch.cuda.synchronize()
    same = all(bytes_equal(a, b) for a, b in zip(snap, dbufs.values()))
    return DecodeResult(out_to_f64(out), pool, pool0, same)


def check_decode(case, res: DecodeResult, want_out, want_state, rows=None, out_tolerance=None,
                 check_untouched=True, verbose=False):
    """Compare a GPU decode with the oracle: pooled and per-(row, v-head)
    relative L1 and every element of the live rows' outputs and states,
    padded rows exact zeros, untouched slots and inputs byte-identical.
    `rows` (an index array) when the oracle ran on a subset of the batch."""
    idx = case.idx if rows is None else case.idx[np.asarray(rows)]
    got_out = res.out if rows is None else res.out[np.asarray(rows)]
    live = idx >= 0
    tol = out_tolerance or out_tol(case)
    assert np.all(got_out[~live] == 0.0), "padded rows must be exact zeros"
    assert np.isfinite(got_out[live]).all(), f"{case.name}: non-finite output"
    check_units(got_out[live], want_out[live], 2, tol, f"{case.name} output")
    atol, rtol = close_tol(case.in_dtype, case.out_dtype)
    if out_tolerance is not None:
        atol, rtol = min(atol, out_tolerance), min(rtol, out_tolerance)
    check_close(got_out[live], want_out[live], atol, rtol, f"{case.name} output")
    r_out = rel_l1(got_out[live], want_out[live])
    got_state = res.pool[torch.from_numpy(idx[live].astype(np.int64)).to(res.pool.device)]
    r_st = _check_state(got_state, want_state[live], case.name, STATE_TOL, case.in_dtype)
    if verbose:
        om, oa = diff_stats(got_out[live], want_out[live])
        print(f"  {case.name}: out rel-L1 {r_out:.3e} max|d| {om:.3e} mean|d| {oa:.3e}; "
              f"state rel-L1 {r_st:.3e}", flush=True)
    if check_untouched and res.pool0 is not None:
        touched = np.zeros(case.num_slots, dtype=bool)
        touched[case.idx[case.idx >= 0]] = True
        untouched = torch.from_numpy(np.nonzero(~touched)[0]).to(res.pool.device)
        if untouched.numel():
            assert bytes_equal(res.pool[untouched], res.pool0[untouched]), \
                f"{case.name}: an untouched slot changed"
    assert res.inputs_unchanged, f"{case.name}: an input buffer was written"
    return r_out, r_st


@dataclass
class PrefillResult:
    out: np.ndarray
    pool: torch.Tensor
    pool0: Optional[torch.Tensor]
    inputs_unchanged: bool


def run_prefill(case: W.PrefillCase, dev, *, sequential: bool = False, keep_pool0=True,
                pool=None, aux: bool = False) -> PrefillResult:
    dbufs, q, k, v = upload_views(case, dev, case.total_tokens)
    snap = [t.clone() for t in dbufs.values()]
    alpha = torch.from_numpy(case.alpha).to(dev)
    dt_bias = torch.from_numpy(case.dt_bias).to(dev)
    ssm_a = torch.from_numpy(case.ssm_a).to(dev)
    beta = torch.from_numpy(case.beta).to(dev)
    cu = torch.from_numpy(case.cu_seqlens).to(dev)
    idx = torch.from_numpy(case.idx).to(dev)
    has_init = torch.from_numpy(case.has_init).to(dev)
    if pool is None:
        pool = torch.from_numpy(case.pool).to(dev)
    pool0 = pool.clone() if keep_pool0 else None
    g = gdn.gate(alpha, dt_bias, ssm_a)
    out = gdn.prefill_varlen(q, k, v, g, beta, pool, cu, scale=case.scale, state_idx=idx,
                             has_initial_state=has_init, l2norm=case.l2norm,
                             l2_eps=case.l2_eps, out_dtype=TORCH_OF[case.out_dtype],
                             sequential=sequential,
                             aux_stream=torch.cuda.Stream() if aux else None)
    torch.cuda.synchronize()
    same = all(bytes_equal(a, b) for a, b in zip(snap, dbufs.values()))
    return PrefillResult(out_to_f64(out), pool, pool0, same)


def check_prefill(case, res: PrefillResult, want_out, want_state, heads=None,
                  out_tolerance=None, state_tolerance=None, verbose=False, check_out=True):
    """Compare a GPU prefill with the oracle (optionally on a subset of
    v-heads): pooled and per-(token, v-head) relative L1 and every element of
    the outputs (unless the caller checks them itself: check_out=False),
    pooled and per-(sequence, v-head) relative L1 and every element of the
    final states, untouched slots and inputs byte-identical."""
    hsel = np.arange(case.hv) if heads is None else np.asarray(heads)
    tol = out_tolerance or out_tol(case)
    st_tol = state_tolerance or STATE_TOL
    got = res.out[:, hsel]
    want = want_out[:, hsel]
    if check_out:
        assert np.isfinite(got).all(), f"{case.name}: non-finite output"
        check_units(got, want, 2, tol, f"{case.name} output")
        atol, rtol = close_tol(case.in_dtype, case.out_dtype)
        if out_tolerance is not None:
            atol, rtol = min(atol, out_tolerance), min(rtol, out_tolerance)
        check_close(got, want, atol, rtol, f"{case.name} output")
    r_out = rel_l1(got, want)
    idx = torch.from_numpy(case.idx.astype(np.int64)).to(res.pool.device)
    got_state = res.pool[idx][:, torch.from_numpy(hsel).to(res.pool.device)]
    r_st = _check_state(got_state, want_state[:, hsel], case.name, st_tol, case.in_dtype)
    if verbose:
        om, oa = diff_stats(got, want)
        sm, sa = diff_stats(got_state.float().cpu().numpy(), want_state[:, hsel])
        print(f"  {case.name}: out rel-L1 {r_out:.3e} max|d| {om:.3e} mean|d| {oa:.3e}; "
              f"state rel-L1 {r_st:.3e} max|d| {sm:.3e} mean|d| {sa:.3e}", flush=True)
    if res.pool0 is not None:
        touched = np.zeros(case.num_slots, dtype=bool)
        touched[case.idx] = True
        untouched = torch.from_numpy(np.nonzero(~touched)[0]).to(res.pool.device)
        if untouched.numel():
            assert bytes_equal(res.pool[untouched], res.pool0[untouched]), \
                f"{case.name}: an untouched slot changed"
    assert res.inputs_unchanged, f"{case.name}: an input buffer was written"
    return r_out, r_st
