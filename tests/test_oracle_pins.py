"""Pins for the CPU oracle: the pages' worked values, closed forms, format
definitions and invariants of the method.  Each test is chosen so that a
plausible mistake in the oracle (a dropped decay, a sign, the old vs updated
state in the output, a transposed state, the GQA head map, eps placement,
the softplus branch) fails at least one of them.  CPU only."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _lnval(s):
    if isinstance(s, str):
        return {"0": 0.0, "ln(0.5)": math.log(0.5)}[s]
    return float(s)


def run_decode(q, k, v, g, beta, S0, scale, *, hk=1, hv=1, l2norm=False, idx=None,
               in_dt=W.F32, pool=None):
    """Tiny f32 decode: q,k [B,hk,dk]; v [B,hv,dv]; g,beta [B,hv]; S0 [B,hv,dv,dk]."""
    q = np.asarray(q, np.float64)
    B, _, dk = q.shape
    dv = np.asarray(v).shape[-1]
    qb = W.encode(q.reshape(B, -1), in_dt)
    kb = W.encode(np.asarray(k, np.float64).reshape(B, -1), in_dt)
    vb = W.encode(np.asarray(v, np.float64).reshape(B, -1), in_dt)
    if pool is None:
        pool = np.ascontiguousarray(np.asarray(S0, np.float32).reshape(B, hv, dv, dk))
    if idx is None:
        idx = np.arange(B, dtype=np.int32)
    return oracle.decode(batch=B, hk=hk, hv=hv, dk=dk, dv=dv, q=qb, q_off=0, q_rs=hk * dk,
                         k=kb, k_off=0, k_rs=hk * dk, v=vb, v_off=0, v_rs=hv * dv,
                         in_dt=in_dt, g=np.asarray(g, np.float64).reshape(B, hv),
                         beta=np.ascontiguousarray(np.asarray(beta, np.float32).reshape(B, hv)),
                         pool=pool, idx=np.asarray(idx, np.int32), scale=scale, l2norm=l2norm)


def run_prefill(q, k, v, g, beta, S0, scale, cu, *, hk=1, hv=1, l2norm=False, idx=None,
                has_init=None, in_dt=W.F32):
    q = np.asarray(q, np.float64)
    T, _, dk = q.shape
    dv = np.asarray(v).shape[-1]
    pool = np.ascontiguousarray(np.asarray(S0, np.float32).reshape(-1, hv, dv, dk))
    return oracle.prefill_varlen(
        cu_seqlens=np.asarray(cu, np.int32), hk=hk, hv=hv, dk=dk, dv=dv,
        q=W.encode(q.reshape(T, hk * dk), in_dt), q_off=0, q_rs=hk * dk,
        k=W.encode(np.asarray(k, np.float64).reshape(T, hk * dk), in_dt), k_off=0, k_rs=hk * dk,
        v=W.encode(np.asarray(v, np.float64).reshape(T, hv * dv), in_dt), v_off=0, v_rs=hv * dv,
        in_dt=in_dt, g=np.asarray(g, np.float64).reshape(T, hv),
        beta=np.ascontiguousarray(np.asarray(beta, np.float32).reshape(T, hv)), pool=pool,
        idx=None if idx is None else np.asarray(idx, np.int32),
        has_init=None if has_init is None else np.asarray(has_init, np.int8),
        scale=scale, l2norm=l2norm)


# ----------------------------------------------------------------------------
# worked values printed on the pages
# ----------------------------------------------------------------------------
def test_decode_single_step_hand_values():
    d = gold("decode_single_step.json")
    out, st = run_decode([[d["q"]]], [[d["k"]]], [[d["v"]]], [[_lnval(d["g"])]], [[d["beta"]]],
                         [[d["S0"]]], d["scale"])
    tol = d["page_tolerance"]
    np.testing.assert_allclose(out[0, 0], d["out"], rtol=tol, atol=0)
    np.testing.assert_allclose(st[0, 0], d["S"], rtol=tol, atol=0)


@pytest.mark.parametrize("dt", [W.BF16, W.F16])
def test_decode_single_step_half_inputs(dt):
    # vllm.cpp 'gdn decode: bf16 q/k/v in, bf16 out, f32 state enforced': the
    # hand case's inputs are exact in bf16 (and binary16), state math stays f32+.
    d = gold("decode_single_step.json")
    out, st = run_decode([[d["q"]]], [[d["k"]]], [[d["v"]]], [[_lnval(d["g"])]], [[d["beta"]]],
                         [[d["S0"]]], d["scale"], in_dt=dt)
    np.testing.assert_allclose(out[0, 0], d["out"], rtol=0.01)
    np.testing.assert_allclose(st[0, 0], d["S"], rtol=1e-12)


def test_prefill_three_token_table():
    d = gold("prefill_three_tokens.json")
    g = [_lnval(x) for x in d["g"]]
    q = np.asarray(d["q"], float)[:, None, :]
    k = np.asarray(d["k"], float)[:, None, :]
    v = np.asarray(d["v"], float)[:, None, :]
    tol = d["page_tolerance"]
    # every prefix of the table: outputs and the state after token t
    for t in range(1, 4):
        out, st = run_prefill(q[:t], k[:t], v[:t], np.array(g[:t])[:, None],
                              np.array(d["beta"][:t])[:, None], [d["S0"]], d["scale"], [0, t])
        for i in range(t):
            np.testing.assert_allclose(out[i, 0], d["per_token"][i]["o"], rtol=tol, atol=1e-15)
        np.testing.assert_allclose(st[0, 0], d["per_token"][t - 1]["S_after"], rtol=tol,
                                   atol=1e-15)


def test_l2norm_values():
    for c in gold("l2norm.json")["cases"]:
        y = oracle.l2norm(np.asarray(c["x"], float), c["eps"])
        np.testing.assert_allclose(y, c["want"], rtol=1e-12, atol=0)
        assert np.all(np.isfinite(y))


def test_l2norm_unit_rows():
    x = np.random.default_rng(3).normal(size=(50, 128))
    y = oracle.l2norm(x, 1e-6)
    n = np.sqrt((y * y).sum(-1))
    # sum of squares is s/(s+eps): within eps/s of one
    np.testing.assert_allclose(n, 1.0, atol=1e-7)
    # direction unchanged (same sign pattern and ratios)
    np.testing.assert_allclose(y * np.linalg.norm(x, axis=-1, keepdims=True) / x,
                               n[:, None] * np.ones_like(x), rtol=1e-6)


# ----------------------------------------------------------------------------
# storage decoders vs the format definitions (library routine on exact cases)
# ----------------------------------------------------------------------------
def test_half_and_bfloat_decoders():
    bits16 = np.array([0x3C00, 0xC000, 0x7BFF, 0x0001, 0x0400, 0x03FF, 0x3555, 0x8000,
                       0x7C00, 0xFC00], dtype=np.uint16)
    want = bits16.view(np.float16).astype(np.float64)
    got = [oracle.decode_value(bits16, W.F16, i) for i in range(len(bits16))]
    np.testing.assert_array_equal(got, want)
    assert got[3] == 2.0 ** -24 and got[4] == 2.0 ** -14
    assert math.isnan(oracle.decode_value(np.array([0x7E00], np.uint16), W.F16, 0))
    bb = np.array([0x3F80, 0x4049, 0xC2F7, 0x0001, 0xFF80], dtype=np.uint16)
    got = [oracle.decode_value(bb, W.BF16, i) for i in range(len(bb))]
    want = (bb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(got, want)
    assert got[0] == 1.0 and got[1] == 3.140625 and got[2] == -123.5


def test_bf16_encoder_round_to_nearest_even_and_nan():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, np.nan,
                  3.4e38], np.float32)
    b = W.f32_to_bf16_bits(x)
    assert b[0] == 0x3F80
    assert b[1] == 0x3F80          # tie -> even
    assert b[2] == 0x3F82          # tie -> even (up)
    assert b[3] == 0x3F81          # above the tie -> up
    assert b[4] & 0x7FC0 == 0x7FC0  # NaN stays NaN, quiet bit set
    assert b[5] == 0x7F80          # rounds past the largest finite -> inf


# ----------------------------------------------------------------------------
# gate: closed forms and the page's branch fixture
# ----------------------------------------------------------------------------
def test_softplus_closed_forms():
    sp = oracle.softplus
    assert abs(sp([0.0])[0] - math.log(2.0)) <= 1e-16
    # softplus(ln(e-1)) = log(1 + e - 1) = 1
    assert abs(sp([math.log(math.e - 1.0)])[0] - 1.0) <= 2e-16
    # softplus(x) - softplus(-x) = x, away from the branch
    x = np.linspace(-19.5, 19.5, 79)
    np.testing.assert_allclose(sp(x) - sp(-x), x, atol=1e-13, rtol=0)
    # tiny tail: log1p(e^-30) = e^-30 (1 - e^-30/2 + ...)
    assert abs(sp([-30.0])[0] / math.exp(-30.0) - 1.0) < 1e-12
    # at the threshold the non-branch side is used (x > 20 is strict)
    assert sp([20.0])[0] == pytest.approx(20.0 + math.log1p(math.exp(-20.0)), rel=1e-15)
    assert sp([20.0])[0] != 20.0
    # above the threshold: exactly x; finite far past the f32 exp overflow
    big = np.array([20.0000001, 88.5, 120.0, 1000.0])
    np.testing.assert_array_equal(sp(big), big)


def test_gate_branch_fixture():
    d = gold("gate_branch.json")
    n = d["H_V"]
    rng = np.random.default_rng(11)
    alpha = np.where(np.arange(n) % 3 == 0, 22.0 + 6.0 * (np.arange(n) % 17),
                     rng.normal(0, 3.0, n)).astype(np.float32)
    dt = (rng.normal(0, 0.5, n)).astype(np.float32)
    a = (-(np.abs(rng.normal(0, 1, n)) + 0.1)).astype(np.float32)
    x = alpha.astype(np.float64) + dt.astype(np.float64)
    assert (x > d["threshold"]).any() and (x > d["f32_exp_overflow_near"]).any()
    g = oracle.gate(alpha[None, :], W.F32, dt, a)[0]
    assert np.all(np.isfinite(g))
    # the branch: g = x * ssm_a exactly in f64 where x > 20
    big = x > 20.0
    np.testing.assert_array_equal(g[big], x[big] * a[big].astype(np.float64))
    # below the branch, softplus(x) = -g/ssm_a lies strictly between max(x,0) and max(x,0)+ln2
    sp = g[~big] / a[~big].astype(np.float64)
    assert np.all(sp > np.maximum(x[~big], 0.0)) and np.all(sp <= np.maximum(x[~big], 0) + math.log(2) + 1e-15)
    # ssm_a < 0 => exp(g) < 1 for every head: the state decays
    assert np.all(np.exp(g) < 1.0)


def test_gate_on_configured_inputs_is_finite_and_decays():
    case = W.decode_b256()
    g = oracle.gate(case.alpha, W.F32, case.dt_bias, case.ssm_a)
    x = case.alpha.astype(np.float64) + case.dt_bias.astype(np.float64)
    assert (x > 88).any() and x.max() <= 121.5
    assert np.all(np.isfinite(g)) and np.all(g < 0) and np.all(np.exp(g) < 1)


def test_gate_row_stride_and_half_alpha():
    rng = np.random.default_rng(5)
    rows, hv, stride = 7, 5, 9
    alpha = rng.normal(0, 3, (rows, stride)).astype(np.float32)
    dt = rng.normal(0, 0.5, hv).astype(np.float32)
    a = -np.exp(rng.uniform(0, 2, hv)).astype(np.float32)
    g_strided = oracle.gate(alpha, W.F32, dt, a, alpha_row_stride=stride)
    g_compact = oracle.gate(np.ascontiguousarray(alpha[:, :hv]), W.F32, dt, a)
    np.testing.assert_array_equal(g_strided, g_compact)
    hb = W.encode(alpha[:, :hv], W.BF16)
    g_bf = oracle.gate(hb, W.BF16, dt, a)
    g_ref = oracle.gate(np.ascontiguousarray(W.decode_to_f32(hb, W.BF16)), W.F32, dt, a)
    np.testing.assert_array_equal(g_bf, g_ref)


# ----------------------------------------------------------------------------
# invariants of the recurrence
# ----------------------------------------------------------------------------
def r32(x):
    """values exactly representable in f32 (what the oracle reads back)"""
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def _rand_head(rng, dk, dv, B=1, hv=1, hk=1):
    q = r32(rng.normal(size=(B, hk, dk)))
    k = r32(rng.normal(size=(B, hk, dk)))
    v = r32(rng.normal(size=(B, hv, dv)))
    S0 = rng.normal(0, 0.3, size=(B, hv, dv, dk)).astype(np.float32)
    return q, k, v, S0


def test_beta0_g0_leaves_state_and_reads_it():
    rng = np.random.default_rng(7)
    q, k, v, S0 = _rand_head(rng, 8, 6)
    out, st = run_decode(q, k, v, [[0.0]], [[0.0]], S0, 0.3, l2norm=True)
    np.testing.assert_array_equal(st, S0.astype(np.float64))
    qn = q[0, 0] / np.sqrt((q[0, 0] ** 2).sum() + 1e-6) * 0.3
    np.testing.assert_allclose(out[0, 0], S0[0, 0].astype(np.float64) @ qn, rtol=1e-13)


def test_beta0_pure_decay_shrinks_norm_each_step():
    rng = np.random.default_rng(8)
    T = 6
    q = r32(rng.normal(size=(T, 1, 8)))
    k = r32(rng.normal(size=(T, 1, 8)))
    v = r32(rng.normal(size=(T, 1, 4)))
    S0 = rng.normal(size=(1, 1, 4, 8)).astype(np.float32)
    g = -np.abs(rng.normal(size=(T, 1))) - 0.01
    norms = []
    for t in range(T + 1):
        _, st = run_prefill(q[:t], k[:t], v[:t], g[:t], np.zeros((t, 1)), S0, 0.5, [0, t])
        norms.append(np.linalg.norm(st))
        np.testing.assert_allclose(st[0, 0], math.exp(g[:t].sum()) * S0[0, 0].astype(np.float64), rtol=1e-13)
    assert all(b < a for a, b in zip(norms, norms[1:]))


def test_beta1_writes_value_at_key():
    # delta rule with beta = 1 and a unit key overwrites the value stored at k:
    # S_new k = decay S k + (v - decay S k)(k.k) = v
    rng = np.random.default_rng(9)
    q, k, v, S0 = _rand_head(rng, 16, 12)
    for g in (0.0, -0.7, -25.0):
        _, st = run_decode(q, k, v, [[g]], [[1.0]], S0, 0.25, l2norm=True)
        kn = k[0, 0] / np.sqrt((k[0, 0] ** 2).sum() + 1e-6)
        kk = (kn * kn).sum()
        want = v[0, 0] * kk + math.exp(g) * (S0[0, 0].astype(np.float64) @ kn) * (1 - kk)
        np.testing.assert_allclose(st[0, 0] @ kn, want, rtol=1e-11, atol=1e-12)


def test_output_reads_updated_state():
    # o = S_new q, not S_old q: with q = k (unit), beta = 1, g = 0: o = scale * v
    rng = np.random.default_rng(10)
    k = rng.normal(size=(1, 1, 8))
    k = r32(k / np.linalg.norm(k))
    kk = (k * k).sum()
    v = r32(rng.normal(size=(1, 1, 5)))
    S0 = rng.normal(size=(1, 1, 5, 8)).astype(np.float32)
    out, _ = run_decode(k, k, v, [[0.0]], [[1.0]], S0, 0.5)
    # S_new k = v (k.k) + S0 k (1 - k.k); k.k = 1 up to f32 rounding of k
    want = 0.5 * (v[0, 0] * kk + (S0[0, 0].astype(np.float64) @ k[0, 0]) * (1 - kk))
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-12)
    np.testing.assert_allclose(out[0, 0], 0.5 * v[0, 0], rtol=1e-6)


def _chunked_wy(q, k, v, g, beta, S0, C):
    """Independent route to the same result: the chunk-parallel (WY) form of the
    gated delta rule, derived from the recurrence.  Rows of Q,K,V are tokens
    (q already scaled, k normalised); S is [dv, dk]."""
    T = q.shape[0]
    S = S0.copy()
    out = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        Q, K, V, gg, bb = q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1]
        G = np.cumsum(gg)
        n = c1 - c0
        E = np.zeros((n, n))
        for i in range(n):
            for j in range(i + 1):
                E[i, j] = math.exp(G[i] - G[j])
        A = np.tril(bb[:, None] * E * (K @ K.T), -1)
        Tm = np.linalg.inv(np.eye(n) + A)
        U = Tm @ (bb[:, None] * (V - np.exp(G)[:, None] * (K @ S.T)))
        out[c0:c1] = np.exp(G)[:, None] * (Q @ S.T) + (E * (Q @ K.T)) @ U
        S = math.exp(G[-1]) * S + (U * np.exp(G[-1] - G)[:, None]).T @ K
    return out, S


@pytest.mark.parametrize("C", [1, 4, 16])
def test_sequential_equals_chunked_form(C):
    rng = np.random.default_rng(12)
    T, dk, dv = 37, 8, 6
    q = r32(rng.normal(size=(T, 1, dk)))
    k = r32(rng.normal(size=(T, 1, dk)))
    v = r32(rng.normal(size=(T, 1, dv)))
    g = -np.abs(rng.normal(size=(T, 1)))
    g[5, 0] = -900.0  # a gate that underflows exp inside a chunk
    beta = rng.uniform(0.05, 0.95, size=(T, 1)).astype(np.float32)
    S0 = rng.normal(0, 0.3, size=(1, 1, dv, dk)).astype(np.float32)
    out, st = run_prefill(q, k, v, g, beta, S0, 0.35, [0, T], l2norm=True)
    kn = k[:, 0] / np.sqrt((k[:, 0] ** 2).sum(-1, keepdims=True) + 1e-6)
    qn = q[:, 0] / np.sqrt((q[:, 0] ** 2).sum(-1, keepdims=True) + 1e-6) * 0.35
    o2, s2 = _chunked_wy(qn, kn, v[:, 0], g[:, 0], beta[:, 0].astype(np.float64),
                         S0[0, 0].astype(np.float64), C)
    np.testing.assert_allclose(out[:, 0], o2, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(st[0, 0], s2, rtol=1e-9, atol=1e-11)


def test_linear_in_state_and_values():
    rng = np.random.default_rng(13)
    T, dk, dv = 9, 6, 5
    q = r32(rng.normal(size=(T, 1, dk))); k = r32(rng.normal(size=(T, 1, dk)))
    va = r32(rng.normal(size=(T, 1, dv))); vb = r32(rng.normal(size=(T, 1, dv)))
    g = -np.abs(rng.normal(size=(T, 1))); beta = rng.uniform(0.1, 0.9, (T, 1))
    Sa = rng.normal(size=(1, 1, dv, dk)).astype(np.float32)
    Sb = rng.normal(size=(1, 1, dv, dk)).astype(np.float32)
    oa, sa = run_prefill(q, k, va, g, beta, Sa, 0.4, [0, T], l2norm=True)
    ob, sb = run_prefill(q, k, vb, g, beta, Sb, 0.4, [0, T], l2norm=True)
    # sums of f32 inputs are exact in f64 only approximately; compare in f64 via pools
    oab, sab = run_prefill(q, k, va + vb, g, beta, (Sa.astype(np.float64) + Sb).astype(np.float32),
                           0.4, [0, T], l2norm=True)
    np.testing.assert_allclose(oab, oa + ob, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(sab, sa + sb, rtol=1e-6, atol=1e-6)


def test_a_run_of_tokens_maps_the_state_affinely():
    """The map that splitting a sequence into segments rests on: over a run of
    tokens the final state is S_in M + S_loc, with M = prod_t decay_t (I -
    beta_t k_t k_t^T) the run's walk of the identity with v = 0 (a dk x dk
    "state") and S_loc its walk from zero.  Both are formed here by the oracle
    itself and checked against its walk from random entry states, with a
    gate that underflows exp inside the run."""
    rng = np.random.default_rng(29)
    T, dk, dv = 23, 8, 5
    q = r32(rng.normal(size=(T, 1, dk)))
    k = r32(rng.normal(size=(T, 1, dk)))
    v = r32(rng.normal(size=(T, 1, dv)))
    g = -np.abs(rng.normal(size=(T, 1)))
    g[7, 0] = -900.0
    beta = rng.uniform(0.05, 0.95, size=(T, 1)).astype(np.float32)
    eye = np.eye(dk, dtype=np.float32)[None, None]
    _, M = run_prefill(q, k, np.zeros((T, 1, dk)), g, beta, eye, 0.3, [0, T], l2norm=True)
    _, S_loc = run_prefill(q, k, v, g, beta, np.zeros((1, 1, dv, dk), np.float32), 0.3, [0, T],
                           l2norm=True)
    M, S_loc = M[0, 0], S_loc[0, 0]
    # M is the product of the per-token maps, taken in token order
    kn = k[:, 0].astype(np.float64)
    kn = kn / np.sqrt((kn ** 2).sum(-1, keepdims=True) + 1e-6)
    P = np.eye(dk)
    for t in range(T):
        P = P @ (math.exp(g[t, 0]) * (np.eye(dk) - float(beta[t, 0]) * np.outer(kn[t], kn[t])))
    np.testing.assert_allclose(M, P, rtol=1e-10, atol=1e-12)
    for trial in range(3):
        S_in = rng.normal(0, 0.5, size=(1, 1, dv, dk)).astype(np.float32)
        _, S_out = run_prefill(q, k, v, g, beta, S_in, 0.3, [0, T], l2norm=True)
        want = S_in[0, 0].astype(np.float64) @ M + S_loc
        np.testing.assert_allclose(S_out[0, 0], want, rtol=1e-10, atol=1e-12)


def test_gqa_ratio3_equals_independent_heads():
    d = gold("gqa_varlen_indexed.json")["gqa"]
    hk, hv, dk, dv = d["hk"], d["hv"], d["dk"], d["dv"]
    q = np.asarray(d["q"]).reshape(1, hk, dk)
    k = np.asarray(d["k"]).reshape(1, hk, dk)
    v = np.array([[0.5 + 0.25 * h, -1.0 + 0.5 * h] for h in range(hv)]).reshape(1, hv, dv)
    g = np.array([-0.1 * (h + 1) for h in range(hv)]).reshape(1, hv)
    beta = np.array([0.1 + 0.1 * h for h in range(hv)]).reshape(1, hv)
    S = np.array([[0.125 * h - 0.0625 * e for e in range(dv * dk)] for h in range(hv)],
                 np.float32).reshape(1, hv, dv, dk)
    out, st = run_decode(q, k, v, g, beta, S, d["scale"], hk=hk, hv=hv)
    for h in range(hv):
        m = h // (hv // hk)
        o1, s1 = run_decode(q[:, m:m + 1], k[:, m:m + 1], v[:, h:h + 1], g[:, h:h + 1],
                            beta[:, h:h + 1], S[:, h:h + 1], d["scale"])
        np.testing.assert_array_equal(out[0, h], o1[0, 0])
        np.testing.assert_array_equal(st[0, h], s1[0, 0])
    # the mapping is grouped: v-head 1 uses q/k head 0, so hv % hk would differ
    o_wrong, _ = run_decode(q[:, 1:2], k[:, 1:2], v[:, 1:2], g[:, 1:2], beta[:, 1:2],
                            S[:, 1:2], d["scale"])
    assert not np.allclose(out[0, 1], o_wrong[0, 0])


def test_varlen_equals_independent_runs():
    d = gold("gqa_varlen_indexed.json")["varlen"]
    T, dk, dv = 5, 2, 2
    t = np.arange(T, dtype=float)
    q = np.stack([0.3 * t - 0.5, 0.9 - 0.2 * t], -1)[:, None]
    k = np.stack([0.7 - 0.3 * t, 0.1 * (t + 1)], -1)[:, None]
    v = np.stack([1.0 - 0.4 * t, -0.5 + 0.3 * t], -1)[:, None]
    g = (-0.05 * (t + 1))[:, None]
    beta = (0.2 + 0.15 * t)[:, None]
    S = np.asarray(d["state"], np.float32).reshape(2, 1, dv, dk)
    cu = d["qsl"]
    out, st = run_prefill(q, k, v, g, beta, S, d["scale"], cu)
    for s in range(2):
        a, b = cu[s], cu[s + 1]
        o1, s1 = run_prefill(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], S[s:s + 1], d["scale"],
                             [0, b - a])
        np.testing.assert_array_equal(out[a:b], o1)
        np.testing.assert_array_equal(st[s], s1[0])


def test_prefill_t1_equals_decode():
    d = gold("gqa_varlen_indexed.json")["t1"]
    args = ([[d["q"]]], [[d["k"]]], [[d["v"]]], [[d["g"]]], [[d["beta"]]],
            np.asarray(d["state"], np.float32).reshape(1, 1, 2, 2), d["scale"])
    od, sd = run_decode(*args)
    op, sp = run_prefill(*args, [0, 1])
    np.testing.assert_array_equal(od, op)
    np.testing.assert_array_equal(sd, sp)


def test_indexed_equals_compact_and_null_rows():
    d = gold("gqa_varlen_indexed.json")["indexed"]
    q = np.asarray(d["q"]).reshape(2, 1, 2); k = np.asarray(d["k"]).reshape(2, 1, 2)
    v = np.asarray(d["v"]).reshape(2, 1, 2)
    g = np.asarray(d["g"]).reshape(2, 1); beta = np.asarray(d["beta"]).reshape(2, 1)
    compact = np.asarray(d["s0"] + d["s1"], np.float32).reshape(2, 1, 2, 2)
    oc, sc = run_decode(q, k, v, g, beta, compact, d["scale"])
    cache = np.full((3, 1, 2, 2), d["sentinel"], np.float32)
    cache[2] = compact[0]
    cache[0] = compact[1]
    oi, si = run_decode(q, k, v, g, beta, None, d["scale"], idx=d["idx"], pool=cache)
    np.testing.assert_array_equal(oi, oc)
    np.testing.assert_array_equal(si, sc)
    # a padded row (idx < 0) gives an exact zero output
    on, sn = run_decode(q, k, v, g, beta, None, d["scale"], idx=[2, -1], pool=cache)
    np.testing.assert_array_equal(on[0], oc[0])
    assert np.all(on[1] == 0.0)


def test_has_init_zero_ignores_slot_contents():
    rng = np.random.default_rng(14)
    q, k, v, _ = _rand_head(rng, 4, 4, B=3)
    g = -np.ones((3, 1)) * 0.2
    beta = np.full((3, 1), 0.5)
    nan_pool = np.full((1, 1, 4, 4), np.nan, np.float32)
    zero_pool = np.zeros((1, 1, 4, 4), np.float32)
    o1, s1 = run_prefill(q, k, v, g, beta, nan_pool, 0.5, [0, 3], has_init=[0])
    o2, s2 = run_prefill(q, k, v, g, beta, zero_pool, 0.5, [0, 3], has_init=[1])
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_zero_length_sequence_passes_state_through():
    rng = np.random.default_rng(15)
    q, k, v, _ = _rand_head(rng, 4, 3, B=2)
    S = rng.normal(size=(2, 1, 3, 4)).astype(np.float32)
    out, st = run_prefill(q, k, v, -np.ones((2, 1)) * 0.1, np.full((2, 1), 0.5), S, 0.5,
                          [0, 0, 2])
    np.testing.assert_array_equal(st[0], S[0].astype(np.float64))


def test_errors():
    rng = np.random.default_rng(16)
    q, k, v, S = _rand_head(rng, 2, 2, B=1, hv=3, hk=2)
    with pytest.raises(oracle.OracleError):   # Hv not a multiple of Hk
        run_decode(q, k, v, -np.ones((1, 3)), np.ones((1, 3)), S, 0.5, hk=2, hv=3)
    q, k, v, S = _rand_head(rng, 2, 2, B=2)
    for bad_scale in (0.0, -1.0, float("nan")):
        with pytest.raises(oracle.OracleError):
            run_decode(q, k, v, -np.ones((2, 1)), np.ones((2, 1)), S, bad_scale)
    pool = np.zeros((2, 1, 2, 2), np.float32)
    for bad_idx in ([0, 0], [0, 2]):          # duplicate, out of range
        with pytest.raises(oracle.OracleError):
            run_decode(q, k, v, -np.ones((2, 1)), np.ones((2, 1)), None, 0.5, idx=bad_idx,
                       pool=pool)


def test_packed_rows_equal_contiguous():
    base = W.make_decode_case("p", 77, batch=5, hk=2, hv=4, dk=16, dv=8, in_dtype=W.F16,
                              out_dtype=W.F16, slots=9, packed_pad=32, null_rows=(3,))
    cont = W.make_decode_case("c", 77, batch=5, hk=2, hv=4, dk=16, dv=8, in_dtype=W.F16,
                              out_dtype=W.F16, slots=9, null_rows=(3,))
    o1, s1 = oracle.decode_case(base)
    o2, s2 = oracle.decode_case(cont)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)
    assert np.all(o1[3] == 0)
    # row sampling gives the same rows
    o3, s3 = oracle.decode_case(base, rows=[4, 1])
    np.testing.assert_array_equal(o3, o1[[4, 1]])
    np.testing.assert_array_equal(s3, s1[[4, 1]])


def test_tiny_prefill_equals_sixty_four_decode_steps():
    pre, _ = W.tiny_prefill_then_decode()
    out, st = oracle.prefill_case(pre)
    g = oracle.gate(pre.alpha, W.F32, pre.dt_bias, pre.ssm_a)
    S = pre.pool.copy()
    for t in range(pre.total_tokens):
        o, s = oracle.decode(batch=1, hk=pre.hk, hv=pre.hv, dk=pre.dk, dv=pre.dv,
                             q=pre.q.buf[t:t + 1], q_off=0, q_rs=pre.q.row_stride,
                             k=pre.k.buf[t:t + 1], k_off=0, k_rs=pre.k.row_stride,
                             v=pre.v.buf[t:t + 1], v_off=0, v_rs=pre.v.row_stride,
                             in_dt=W.F32, g=g[t:t + 1], beta=pre.beta[t:t + 1].copy(),
                             pool=S, idx=np.zeros(1, np.int32), scale=pre.scale)
        np.testing.assert_allclose(o[0], out[t], rtol=1e-5, atol=1e-8)  # f32 state between steps
        S = s.astype(np.float32)
    np.testing.assert_allclose(S[0], st[0], rtol=1e-5, atol=1e-8)


def test_threads_do_not_change_results():
    """The oracle's decode and prefill run independent (row or sequence,
    v-head) units on several host threads; every unit's arithmetic is the same
    whatever the thread count, so the results are bit-identical."""
    pre = W.make_prefill_case("thr", 77, lengths=[9, 0, 33, 2], hk=2, hv=6, dk=16, dv=8,
                              in_dtype=W.BF16, out_dtype=W.BF16, slots=6, has_init=[1, 1, 0, 1])
    dec = W.make_decode_case("thr", 78, batch=5, hk=1, hv=3, dk=16, dv=16, in_dtype=W.F16,
                             out_dtype=W.F16, slots=7, null_rows=(1,))
    n0 = oracle.get_threads()
    try:
        oracle.set_threads(1)
        p1 = oracle.prefill_case(pre)
        d1 = oracle.decode_case(dec)
        oracle.set_threads(5)
        p5 = oracle.prefill_case(pre)
        d5 = oracle.decode_case(dec)
    finally:
        oracle.set_threads(n0)
    for a, b in zip(p1 + d1, p5 + d5):
        assert np.array_equal(a, b)
