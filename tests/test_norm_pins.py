"""Pins for the oracle's gated RMSNorm (vllm.cpp tests/vt/test_ops_gdn.cpp,
"rmsnorm_gated: norm-then-gate, silu and sigmoid activations" and the rank-3
padded-row gate case).  CPU only.  Chosen so that a sum instead of a mean, eps
outside the root, gate-then-norm, the wrong activation or a wrong gate row
stride fails one of them."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def norm(x, z, w, *, eps=0.0, sigmoid=False, z_rs=None, rows=None, hv=1):
    x = np.asarray(x, np.float64)
    dv = x.shape[-1]
    rows = x.size // (hv * dv) if rows is None else rows
    z = np.asarray(z, np.float64)
    return oracle.rmsnorm_gated(x, oracle.F64, z, oracle.F64, hv * dv if z_rs is None else z_rs,
                                np.asarray(w, np.float64), oracle.F64, rows=rows, hv=hv, dv=dv,
                                eps=eps, sigmoid=sigmoid)


def test_hand_values_silu_and_sigmoid():
    g = json.load(open(os.path.join(GOLD, "rmsnorm_gated.json")))
    tol = g["printed_digits_tolerance"]
    ones = np.ones(2)
    big = np.full(2, 60.0)   # sigmoid(60) = 1 to double precision: the bare norm
    normed = norm(g["x"], big, ones, sigmoid=True)[0, 0]   # x / rms, before w and the gate
    np.testing.assert_allclose(normed * np.array(g["w"]), g["normed"], atol=tol)
    silu = norm(g["x"], g["z"], g["w"], eps=g["eps"])[0, 0]
    np.testing.assert_allclose(silu, g["out_silu"], atol=tol)
    sig = norm(g["x"], g["z"], g["w"], eps=g["eps"], sigmoid=True)[0, 0]
    np.testing.assert_allclose(sig, g["out_sigmoid"], atol=tol)


def test_variance_is_a_mean():
    # four equal entries: mean(x^2) = 1 -> normed 1 (a sum would give 0.5)
    y = norm([1.0, 1.0, 1.0, 1.0], [60.0] * 4, [1.0] * 4, sigmoid=True)
    np.testing.assert_allclose(y[0, 0], [1.0] * 4, rtol=1e-15)


def test_eps_inside_the_root():
    # x = [1e-3, 0], eps = 1e-6: 1e-3 / sqrt(5e-7 + 1e-6)
    y = norm([1e-3, 0.0], [60.0, 60.0], [1.0, 1.0], eps=1e-6, sigmoid=True)
    assert y[0, 0, 0] == pytest.approx(1e-3 / math.sqrt(1.5e-6), rel=1e-14)
    assert y[0, 0, 1] == 0.0


def test_norm_then_gate_and_scale_invariance():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(3, 2, 8))
    z = rng.normal(size=(3, 16))
    w = rng.uniform(-1, 1, size=8)
    y = norm(x, z, w, hv=2)
    # a positive scale of x changes nothing when eps = 0
    np.testing.assert_allclose(norm(x * 37.5, z, w, hv=2), y, rtol=1e-13)
    # the closed form, written out with numpy
    zz = z.reshape(3, 2, 8)
    want = x / np.sqrt((x ** 2).mean(-1, keepdims=True)) * w * (zz / (1 + np.exp(-zz)))
    np.testing.assert_allclose(y, want, rtol=1e-12)
    # gate-then-norm differs
    g = x * (zz / (1 + np.exp(-zz)))
    wrong = g / np.sqrt((g ** 2).mean(-1, keepdims=True)) * w
    assert np.abs(wrong - y).max() > 1e-3


def test_silu_zero_gate_and_sigmoid_half():
    y = norm([3.0, 4.0], [0.0, 0.0], [1.0, 1.0])
    assert np.all(y == 0.0)                          # silu(0) = 0
    y = norm([3.0, 4.0], [0.0, 0.0], [1.0, 1.0], sigmoid=True)
    np.testing.assert_allclose(y[0, 0], [0.5 * 3 / math.sqrt(12.5), 0.5 * 4 / math.sqrt(12.5)],
                               rtol=1e-15)


def test_padded_rank3_gate_equals_contiguous_and_skips_padding():
    rng = np.random.default_rng(9101)
    T, hv, dv, pad = 4, 3, 5, 11
    x = rng.normal(size=(T, hv, dv))
    z = rng.normal(size=(T, hv * dv))
    w = rng.normal(size=dv)
    y_c = norm(x, z, w, hv=hv)
    zp = np.full((T, hv * dv + pad), np.nan)        # padding must never be read
    zp[:, :hv * dv] = z
    y_p = norm(x, zp, w, hv=hv, z_rs=hv * dv + pad)
    np.testing.assert_array_equal(y_p, y_c)
    assert np.isfinite(y_p).all()


def test_storage_dtypes_are_decoded():
    import workloads as W
    rng = np.random.default_rng(5)
    x = rng.normal(size=(2, 2, 16)).astype(np.float32)
    z = rng.normal(size=(2, 32)).astype(np.float32)
    w = rng.uniform(-1, 1, size=16).astype(np.float32)
    for dt in (W.BF16, W.F16):
        xs, zs, ws = W.encode(x, dt), W.encode(z, dt), W.encode(w, dt)
        dec = lambda a: W.decode_to_f32(a, dt).astype(np.float64)
        y = oracle.rmsnorm_gated(xs, dt, zs, dt, 32, ws, dt, rows=2, hv=2, dv=16, eps=1e-6)
        want = norm(dec(xs), dec(zs), dec(ws), eps=1e-6, hv=2)
        np.testing.assert_array_equal(y, want)


def test_errors():
    with pytest.raises(oracle.OracleError):
        norm([1.0, 2.0], [1.0], [1.0, 1.0], z_rs=1)          # gate row stride < hv*dv
    with pytest.raises(oracle.OracleError):
        norm([1.0, 2.0], [1.0, 1.0], [1.0, 1.0], eps=-1.0)
