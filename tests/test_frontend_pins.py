"""Pins for the oracle's front-end pieces (vllm.cpp tests/vt/test_ops_gdn.cpp:
"gdn_post_conv fused == composed", the packed in_proj_ba case, GdnGBeta, and
PackedDecodeReference's beta rounded through b's dtype).  CPU only."""
import math

import numpy as np
import pytest

import oracle
import workloads as W


def test_round_through_matches_numpy_and_the_bf16_rule():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # binary16: numpy's float32 -> float16 conversion (nearest, ties to even)
    sel = x[:20000]
    want16 = sel.astype(np.float16).astype(np.float64)
    got16 = np.array([oracle.round_through(v, W.F16) for v in sel])
    np.testing.assert_array_equal(got16, want16)
    # the f16 range edges and subnormals
    edge = np.array([65504.0, 65519.0, 65520.0, 2.0**-24, 2.0**-25, 1.5 * 2.0**-25,
                     2.0**-14 - 2.0**-25, 1.0 + 2.0**-11, 1.0 + 3 * 2.0**-11], np.float32)
    with np.errstate(over="ignore"):
        want_edge = edge.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal([oracle.round_through(v, W.F16) for v in edge], want_edge)
    # bfloat16: the pages' rounding rule as the workloads encoder implements it
    want_b = W.decode_to_f32(W.f32_to_bf16_bits(sel), W.BF16).astype(np.float64)
    got_b = np.array([oracle.round_through(v, W.BF16) for v in sel])
    np.testing.assert_array_equal(got_b, want_b)
    assert oracle.round_through(0.1, W.F32) == float(np.float32(0.1))


def _gb(b_vals, dt, round_beta):
    b = W.encode(np.asarray(b_vals, np.float64).reshape(1, -1), dt)
    hv = b.shape[1]
    a = W.encode(np.zeros((1, hv)), dt)
    g, beta = oracle.gate_beta(a, 0, hv, b, 0, hv, dt, np.zeros(hv, np.float32),
                               np.full(hv, -1.0, np.float32), rows=1, hv=hv,
                               round_beta=round_beta)
    return g[0], beta[0]


def test_beta_values():
    _, beta = _gb([0.0, 30.0, -1.0, 1.0], W.F32, False)
    assert beta[0] == 0.5
    assert beta[1] == 1.0                       # 1 - 9.4e-14 rounds to 1 in binary32
    assert beta[2] == pytest.approx(1.0 / (1.0 + math.e), rel=1e-7)
    assert beta[3] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-7)
    # rounded through bfloat16: sigmoid(1) = 0.7310586 -> 187/256
    _, beta = _gb([1.0, 0.0], W.BF16, True)
    assert beta[0] == 187 / 256 and beta[1] == 0.5
    # ... and through binary16: 0.7310586 -> 1497/2048
    _, beta = _gb([1.0], W.F16, True)
    assert beta[0] == 1497 / 2048
    # without the rounding, a bf16 b is only widened
    _, beta = _gb([1.0], W.BF16, False)
    assert beta[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-7)


def test_gate_half_equals_oracle_gate():
    rng = np.random.default_rng(4)
    a = rng.normal(0, 5, size=(6, 4)).astype(np.float32)
    b = rng.normal(size=(6, 4)).astype(np.float32)
    dtb = rng.normal(size=4).astype(np.float32)
    ssa = -np.exp(rng.uniform(0, 2, size=4)).astype(np.float32)
    g, _ = oracle.gate_beta(a, 0, 4, b, 0, 4, W.F32, dtb, ssa, rows=6, hv=4)
    np.testing.assert_array_equal(g, oracle.gate(a, W.F32, dtb, ssa))


def test_merged_ba_view_with_canaries_equals_separate_arrays():
    rng = np.random.default_rng(7)
    rows, hv, prefix, suffix = 5, 6, 1, 3
    width = prefix + 2 * hv + suffix
    a = rng.uniform(-1, 1, size=(rows, hv))
    b = rng.uniform(-1, 1, size=(rows, hv))
    parent = np.full((rows, width), np.nan)          # canaries that must never be read
    parent[:, prefix:prefix + hv] = b
    parent[:, prefix + hv:prefix + 2 * hv] = a
    dtb = rng.normal(size=hv).astype(np.float32)
    ssa = -np.exp(rng.uniform(0, 1, size=hv)).astype(np.float32)
    for dt in (W.F32, W.BF16, W.F16):
        pb = W.encode(parent, dt)
        sa, sb = W.encode(a, dt), W.encode(b, dt)
        for rb in (False, True):
            g1, b1 = oracle.gate_beta(pb, prefix + hv, width, pb, prefix, width, dt, dtb, ssa,
                                      rows=rows, hv=hv, round_beta=rb)
            g2, b2 = oracle.gate_beta(sa, 0, hv, sb, 0, hv, dt, dtb, ssa, rows=rows, hv=hv,
                                      round_beta=rb)
            assert np.isfinite(g1).all() and np.isfinite(b1).all()
            np.testing.assert_array_equal(g1, g2)
            np.testing.assert_array_equal(b1, b2)


def test_post_conv_equals_composed_ops():
    rng = np.random.default_rng(7100)
    T, hk, hv, dk, dv = 5, 2, 6, 16, 8
    cd = 2 * hk * dk + hv * dv
    pad = 3
    conv = np.full((T, cd + pad), np.nan)            # row padding never read
    conv[:, :cd] = rng.uniform(-1.5, 1.5, size=(T, cd))
    a = rng.uniform(-1, 1, size=(T, hv)).astype(np.float32)
    b = rng.uniform(-1, 1, size=(T, hv)).astype(np.float32)
    dtb = rng.uniform(-1, 1, size=hv).astype(np.float32)
    ssa = -np.exp(rng.uniform(-1, 1, size=hv)).astype(np.float32)
    for dt in (W.F32, W.BF16):
        cs = W.encode(conv, dt)
        q, k, v, g, beta = oracle.post_conv(cs, dt, cd + pad, a, 0, hv, b, 0, hv, W.F32, dtb,
                                            ssa, T=T, hk=hk, hv=hv, dk=dk, dv=dv)
        x = W.decode_to_f32(cs, dt).astype(np.float64)[:, :cd]
        qr = x[:, :hk * dk].reshape(T, hk, dk)
        kr = x[:, hk * dk:2 * hk * dk].reshape(T, hk, dk)
        np.testing.assert_array_equal(q, oracle.l2norm(qr, 1e-6))
        np.testing.assert_array_equal(k, oracle.l2norm(kr, 1e-6))
        np.testing.assert_array_equal(v, x[:, 2 * hk * dk:].reshape(T, hv, dv))
        g2, b2 = oracle.gate_beta(a, 0, hv, b, 0, hv, W.F32, dtb, ssa, rows=T, hv=hv)
        np.testing.assert_array_equal(g, g2)
        np.testing.assert_array_equal(beta, b2)
        np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-5)
        # q and k come from different columns (a swapped split would pass the norm check)
        assert not np.allclose(q, k)
