"""Pins for the oracle's depthwise causal conv1d (vllm.cpp tests/vt/test_ops_gdn.cpp,
the causal_conv1d_fwd / causal_conv1d_update cases).  CPU only.  Chosen so
that a flipped tap order, the activation applied to the stored state, a state
that keeps the wrong end, bias dropped, or a window leaking across sequences
fails one of them."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")
F32 = W.F32


def gold():
    return json.load(open(os.path.join(GOLD, "conv1d.json")))


def fwd(x, w, state, cu, *, bias=None, has_init=None, silu=True, idx=None, state_len=None):
    x = np.asarray(x, np.float32)
    T, C = x.shape
    w = np.asarray(w, np.float32)
    K = w.shape[1]
    state = np.asarray(state, np.float32)
    sl = state.shape[-1] if state_len is None else state_len
    return oracle.conv1d_fwd(cu_seqlens=cu, C=C, K=K, x=x, x_dt=F32, x_rs=C, w=w,
                             bias=None if bias is None else np.asarray(bias, np.float32),
                             state=state, st_dt=F32, state_len=sl, idx=idx, has_init=has_init,
                             silu=silu)


def test_fwd_hand_values():
    g = gold()
    f, tol = g["fwd"], g["printed_digits_tolerance"]
    x = np.array(f["x"]).reshape(2, 1)
    w = np.array([f["w"]])
    st = np.array(f["state"]).reshape(1, 1, 2)
    out, s = fwd(x, w, st, [0, 2], bias=[f["bias"]], silu=False)
    np.testing.assert_array_equal(out[:, 0], f["out_linear"])
    out, s = fwd(x, w, st, [0, 2], bias=[f["bias"]], silu=True)
    np.testing.assert_allclose(out[:, 0], f["out_silu"], atol=tol)
    np.testing.assert_array_equal(s[0, 0], f["state_after"])     # raw inputs, not silu'd


def test_fwd_short_sequence_write_back():
    h = gold()["short"]
    x = np.array(h["x"]).reshape(1, 1)
    w = np.array([h["w"]])
    st = np.array(h["state"]).reshape(1, 1, 3)
    out, s = fwd(x, w, st, [0, 1], has_init=[1], silu=False)
    assert out[0, 0] == h["out"][0]
    np.testing.assert_array_equal(s[0, 0], h["state_after_with_init"])
    out, s = fwd(x, w, st, [0, 1], has_init=[0], silu=False)
    np.testing.assert_array_equal(s[0, 0], h["state_after_without_init"])


def test_update_hand_values():
    u = gold()["update"]
    out, s, wr = oracle.conv1d_update(batch=1, C=1, K=3, x=np.array([u["x"]], np.float32),
                                      x_dt=F32, x_rs=1, w=np.array([u["w"]], np.float32),
                                      bias=np.array([u["bias"]], np.float32),
                                      state=np.array(u["state"], np.float32).reshape(1, 1, 2),
                                      st_dt=F32, state_len=2)
    assert out[0, 0] == pytest.approx(u["out_silu"], abs=1e-8)
    np.testing.assert_array_equal(s[0, 0], u["state_after"])
    assert wr[0]


def test_fwd_equals_numpy_convolution_from_zero_state():
    rng = np.random.default_rng(3)
    T, C, K = 23, 5, 4
    x = rng.normal(size=(T, C)).astype(np.float32)
    w = rng.normal(size=(C, K)).astype(np.float32)
    b = rng.normal(size=C).astype(np.float32)
    out, s = fwd(x, w, np.zeros((1, C, K - 1)), [0, T], bias=b, has_init=[0], silu=False)
    for c in range(C):
        # y[t] = sum_j w[j] x[t - (K-1) + j]: a full convolution with the flipped taps
        want = np.convolve(x[:, c].astype(np.float64), w[c, ::-1].astype(np.float64))[:T] + b[c]
        np.testing.assert_allclose(out[:, c], want, rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(s[0, c], x[T - (K - 1):, c])


def test_update_chain_equals_fwd():
    rng = np.random.default_rng(4)
    T, C, K = 6, 3, 4
    x = rng.normal(size=(T, C)).astype(np.float32)
    w = rng.normal(size=(C, K)).astype(np.float32)
    st0 = rng.normal(size=(1, C, K - 1)).astype(np.float32)
    out_f, st_f = fwd(x, w, st0, [0, T], silu=True)
    st = st0
    for t in range(T):
        o, s, _ = oracle.conv1d_update(batch=1, C=C, K=K, x=x[t:t + 1], x_dt=F32, x_rs=C, w=w,
                                       bias=None, state=st, st_dt=F32, state_len=K - 1)
        np.testing.assert_allclose(o[0], out_f[t], rtol=1e-12)
        st = s.astype(np.float32)
    np.testing.assert_array_equal(st[0], st_f[0])


def test_varlen_equals_independent_runs_and_indexed_slots():
    rng = np.random.default_rng(5)
    lengths, C, K = [5, 1, 0, 9], 4, 4
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = rng.normal(size=(T, C)).astype(np.float32)
    w = rng.normal(size=(C, K)).astype(np.float32)
    b = rng.normal(size=C).astype(np.float32)
    slots = 7
    st = rng.normal(size=(slots, C, K - 1)).astype(np.float32)
    idx = np.array([6, 0, 3, 2], np.int32)
    hi = np.array([1, 0, 1, 1], np.int8)
    out, s = fwd(x, w, st, cu, bias=b, has_init=hi, idx=idx)
    for i, L in enumerate(lengths):
        a0 = cu[i]
        o1, s1 = fwd(x[a0:a0 + L], w, st[idx[i]:idx[i] + 1], [0, L], bias=b, has_init=[hi[i]])
        np.testing.assert_array_equal(out[a0:a0 + L], o1)
        np.testing.assert_array_equal(s[i], s1[0])
    np.testing.assert_array_equal(s[2], st[3])       # zero-length: state passes through


def test_widened_cache_uses_the_leading_window():
    rng = np.random.default_rng(6)
    T, C, K, extra = 4, 2, 3, 2
    x = rng.normal(size=(T, C)).astype(np.float32)
    w = rng.normal(size=(C, K)).astype(np.float32)
    narrow = rng.normal(size=(1, C, K - 1)).astype(np.float32)
    wide = np.full((1, C, K - 1 + extra), np.nan, np.float32)   # extra taps never read
    wide[:, :, :K - 1] = narrow
    o1, s1 = fwd(x, w, narrow, [0, T])
    o2, s2 = fwd(x, w, wide, [0, T])
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_update_null_slot_and_padded_rows():
    rng = np.random.default_rng(7)
    B, C, K, pad = 3, 4, 4, 5
    x = np.full((B, C + pad), np.nan, np.float32)                # padded rows: canaries
    x[:, :C] = rng.normal(size=(B, C))
    w = rng.normal(size=(C, K)).astype(np.float32)
    st = rng.normal(size=(4, C, K - 1)).astype(np.float32)
    out, s, wr = oracle.conv1d_update(batch=B, C=C, K=K, x=x, x_dt=F32, x_rs=C + pad, w=w,
                                      bias=None, state=st, st_dt=F32, state_len=K - 1,
                                      idx=np.array([3, -1, 0], np.int32))
    assert list(wr) == [True, False, True]
    assert np.isfinite(out[[0, 2]]).all()
    o2, _, _ = oracle.conv1d_update(batch=1, C=C, K=K, x=np.ascontiguousarray(x[2:3, :C]),
                                    x_dt=F32, x_rs=C, w=w, bias=None, state=st[0:1], st_dt=F32,
                                    state_len=K - 1)
    np.testing.assert_array_equal(out[2], o2[0])


def test_k1_has_no_state():
    x = np.array([[2.0, -1.0]], np.float32)
    w = np.array([[3.0], [0.5]], np.float32)
    out, s = fwd(x, w, np.zeros((1, 2, 0)), [0, 1], bias=[1.0, 0.0], silu=False)
    np.testing.assert_array_equal(out[0], [7.0, -0.5])
    assert s.shape == (1, 2, 0)


def test_errors():
    x = np.zeros((2, 1), np.float32)
    w = np.ones((1, 3), np.float32)
    with pytest.raises(oracle.OracleError):
        fwd(x, w, np.zeros((1, 1, 2)), [0, 2], state_len=1)            # state row too short
    with pytest.raises(oracle.OracleError):
        fwd(x, w, np.zeros((2, 1, 2)), [0, 1, 2], idx=np.array([1, 1], np.int32))  # duplicate
