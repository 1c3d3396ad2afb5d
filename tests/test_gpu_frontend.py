"""GPU parity of the front-end pieces (vllm.cpp tests/vt/test_ops_gdn.cpp:
GdnGBeta and the packed in_proj_ba case, "gdn_post_conv fused == composed",
and PackedDecodeReference's raw-b beta): g and beta from raw a/b views of a
merged row, the post-conv split + norm, and decode reading the conv output
row and the merged b|a row directly.  The NaN canaries around every view
must never be read."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
import linear_attention_recurrence_gdn_amd as gdn
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def ba_views(ba: W.MergedBA, rows, hv, dev):
    t = H.to_dev(ba.buf, ba.dtype, dev).reshape(-1)
    a = t.as_strided((rows, hv), (ba.row_stride, 1), ba.a_off)
    b = t.as_strided((rows, hv), (ba.row_stride, 1), ba.b_off)
    return t, a, b


@pytest.mark.parametrize("rounded", [False, True], ids=["sigmoid", "rounded"])
@pytest.mark.parametrize("dt", [W.F32, W.BF16, W.F16], ids=["f32", "bf16", "f16"])
def test_gate_beta_from_merged_row(dev, dt, rounded):
    announce(f"gate_beta {W.DTYPE_NAMES[dt]} rounded={rounded}")
    rng = np.random.default_rng(31)
    rows, hv = 77, 24
    alpha, dt_bias, ssm_a = W.gate_inputs(rng, rows, hv, large_every_third=True,
                                          head0_offset=0.0, a_log_hi=2.0)
    ba = W.merged_ba(31, alpha, dt)
    parent, a, b = ba_views(ba, rows, hv, dev)
    p0 = parent.clone()
    g, beta = gdn.gate_beta(a, b, torch.from_numpy(dt_bias).to(dev),
                            torch.from_numpy(ssm_a).to(dev), rounded=rounded)
    torch.cuda.synchronize()
    wg, wb = oracle.gate_beta(ba.buf, ba.a_off, ba.row_stride, ba.buf, ba.b_off, ba.row_stride,
                              dt, dt_bias, ssm_a, rows=rows, hv=hv, round_beta=rounded)
    gg, gb = g.cpu().numpy().astype(np.float64), beta.cpu().numpy().astype(np.float64)
    assert np.isfinite(gg).all() and np.isfinite(gb).all()
    assert H.rel_l1(gg, wg) <= 1e-6
    if rounded and dt != W.F32:
        # a value decided by rounding: equal except where the f32 sigmoid sits on a tie
        assert np.mean(gb == wb) >= 0.999
        assert np.max(np.abs(gb - wb)) <= 2.0 ** -8
    else:
        assert np.max(np.abs(gb - wb)) <= 2e-7
    assert H.bytes_equal(parent, p0)


@pytest.mark.parametrize("spec", [
    # (T, hk, hv, dk, dv, conv dtype, out dtype, row padding)
    (5, 2, 6, 128, 128, W.F32, W.F32, 0),
    (24, 16, 32, 128, 128, W.BF16, W.BF16, 8),
    (3, 4, 4, 300, 128, W.BF16, W.F32, 5),
    (1, 1, 2, 64, 64, W.F16, W.F16, 0),
    (17, 4, 8, 128, 128, W.F32, W.BF16, 0),
    # 16-byte lanes: a head on 64 lanes, on one lane, ragged v widths
    (6, 2, 4, 512, 64, W.BF16, W.F16, 0),
    (9, 3, 3, 8, 24, W.F16, W.F32, 0),
    (7, 2, 2, 256, 12, W.F32, W.F16, 0),
    (300, 16, 32, 128, 128, W.BF16, W.BF16, 0),
    # a row stride that is not a multiple of 16 bytes: one element per lane
    (4, 16, 32, 128, 128, W.BF16, W.BF16, 5),
], ids=lambda s: "T{}-hk{}-hv{}-dk{}-dv{}-{}-{}-pad{}".format(
    s[0], s[1], s[2], s[3], s[4], W.DTYPE_NAMES[s[5]], W.DTYPE_NAMES[s[6]], s[7]))
def test_post_conv(dev, spec):
    T, hk, hv, dk, dv, cdt, odt, pad = spec
    announce(f"post_conv {spec}")
    rng = np.random.default_rng(T * 31 + dk)
    width = 2 * hk * dk + hv * dv
    conv = W.nan_fill((T, width + pad), cdt)
    conv[:, :width] = W.encode(rng.uniform(-1.5, 1.5, size=(T, width)), cdt)
    alpha = rng.uniform(-1, 1, size=(T, hv)).astype(np.float32)
    dt_bias = rng.uniform(-1, 1, size=hv).astype(np.float32)
    ssm_a = (-np.exp(rng.uniform(-1, 1, size=hv))).astype(np.float32)
    ba = W.merged_ba(T, alpha, W.BF16, b_range=1.0)
    cd = H.to_dev(conv, cdt, dev)
    c0 = cd.clone()
    _, a, b = ba_views(ba, T, hv, dev)
    q, k, v, g, beta = gdn.post_conv(cd, a, b, torch.from_numpy(dt_bias).to(dev),
                                     torch.from_numpy(ssm_a).to(dev), hk=hk, dk=dk, dv=dv,
                                     out_dtype=H.TORCH_OF[odt])
    torch.cuda.synchronize()
    wq, wk, wv, wg, wb = oracle.post_conv(conv, cdt, width + pad, ba.buf, ba.a_off,
                                          ba.row_stride, ba.buf, ba.b_off, ba.row_stride,
                                          W.BF16, dt_bias, ssm_a, T=T, hk=hk, hv=hv, dk=dk,
                                          dv=dv)
    tol = H.OUT_TOL_F32 if odt == W.F32 else H.OUT_TOL_HALF
    for name, got, want in (("q", q, wq), ("k", k, wk)):
        gv = H.out_to_f64(got)
        assert np.isfinite(gv).all()
        r = H.rel_l1(gv, want)
        assert r <= tol, f"{name}: rel-L1 {r:.3e}"
    # v is a conversion: exactly the nearest value in the output format
    want_v = W.decode_to_f32(W.encode(wv, odt), odt).astype(np.float64)
    np.testing.assert_array_equal(H.out_to_f64(v), want_v)
    assert H.rel_l1(g.cpu().numpy(), wg) <= 1e-6
    assert np.max(np.abs(beta.cpu().numpy() - wb)) <= 2e-7
    assert H.bytes_equal(cd, c0)


@pytest.mark.parametrize("spec", [
    # (batch, hk, hv, dk, dv, in dtype, a/b dtype, out, null rows)
    (6, 2, 4, 128, 128, W.BF16, W.BF16, W.BF16, (2,)),
    (5, 2, 6, 128, 128, W.F32, W.F32, W.F32, ()),
    (4, 1, 3, 64, 64, W.F16, W.F16, W.F32, (0,)),
    (7, 2, 4, 128, 72, W.BF16, W.F32, W.BF16, ()),
], ids=lambda s: "B{}-hv{}-dk{}-dv{}-{}-ab{}".format(s[0], s[2], s[3], s[4],
                                                     W.DTYPE_NAMES[s[5]], W.DTYPE_NAMES[s[6]]))
def test_decode_from_conv_row_and_raw_ba(dev, spec):
    """The fused front-end of decode: q|k|v straight from the conv output row
    (padded with NaN), a and raw b straight from the merged b|a row."""
    B, hk, hv, dk, dv, ind, abd, outd, nulls = spec
    announce(f"decode from conv row + raw b|a {spec}")
    case = W.make_decode_case("fe", 5100 + B * dv, batch=B, hk=hk, hv=hv, dk=dk, dv=dv,
                              in_dtype=ind, out_dtype=outd, slots=B + 3, packed_pad=32,
                              null_rows=nulls, large_every_third=True)
    ba = W.merged_ba(5100 + B, case.alpha, abd)
    dbufs, q, k, v = H.upload_views(case, dev, B)
    _, a, b = ba_views(ba, B, hv, dev)
    t = lambda x: torch.from_numpy(x).to(dev)
    pool = t(case.pool)
    pool0 = pool.clone()
    idx = t(case.idx)
    out = gdn.decode(q, k, v, a, t(case.dt_bias), t(case.ssm_a), b, pool, idx,
                     scale=case.scale, out_dtype=H.TORCH_OF[outd], beta_raw=True)
    torch.cuda.synchronize()
    g, beta = oracle.gate_beta(ba.buf, ba.a_off, ba.row_stride, ba.buf, ba.b_off, ba.row_stride,
                               abd, case.dt_bias, case.ssm_a, rows=B, hv=hv, round_beta=True)
    want_out, want_state = oracle.decode(
        batch=B, hk=hk, hv=hv, dk=dk, dv=dv, q=case.q.buf, q_off=case.q.offset,
        q_rs=case.q.row_stride, k=case.k.buf, k_off=case.k.offset, k_rs=case.k.row_stride,
        v=case.v.buf, v_off=case.v.offset, v_rs=case.v.row_stride, in_dt=ind, g=g,
        beta=beta.astype(np.float32), pool=case.pool, idx=case.idx, scale=case.scale)
    res = H.DecodeResult(H.out_to_f64(out), pool, pool0, True)
    H.check_decode(case, res, want_out, want_state)


@pytest.mark.parametrize("sequential", [True, False], ids=["sequential", "default"])
def test_prefill_from_conv_rows_and_gate_beta(dev, sequential):
    """Prefill reading q|k|v straight from padded conv output rows, with g and
    beta from gdn_gate_beta over a merged b|a row."""
    announce(f"prefill from conv rows + gate_beta sequential={sequential}")
    lengths, hk, hv, dk, dv, dt, pad = [70, 1, 130, 64], 2, 4, 128, 128, W.BF16, 8
    T = sum(lengths)
    rng = np.random.default_rng(5151)
    width = 2 * hk * dk + hv * dv
    conv = W.nan_fill((T, width + pad), dt)
    conv[:, :width] = W.encode(rng.normal(size=(T, width)), dt)
    alpha, dt_bias, ssm_a = W.gate_inputs(rng, T, hv, large_every_third=False,
                                          head0_offset=0.0, a_log_hi=2.0)
    ba = W.merged_ba(5151, alpha, dt)
    slots = len(lengths) + 2
    pool = W.make_pool(5151, slots, hv, dv, dk, 0.05)
    idx = rng.permutation(slots)[:len(lengths)].astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    scale = float(np.float32(1.0 / np.sqrt(dk)))
    t = lambda x: torch.from_numpy(x).to(dev)
    cd = H.to_dev(conv, dt, dev).reshape(-1)
    stride = width + pad
    q = cd.as_strided((T, hk, dk), (stride, dk, 1), 0)
    k = cd.as_strided((T, hk, dk), (stride, dk, 1), hk * dk)
    v = cd.as_strided((T, hv, dv), (stride, dv, 1), 2 * hk * dk)
    _, a, b = ba_views(ba, T, hv, dev)
    g, beta = gdn.gate_beta(a, b, t(dt_bias), t(ssm_a))
    dpool = t(pool)
    out = gdn.prefill_varlen(q, k, v, g, beta, dpool, t(cu), scale=scale, state_idx=t(idx),
                             out_dtype=torch.bfloat16, sequential=sequential)
    torch.cuda.synchronize()
    wg, wb = oracle.gate_beta(ba.buf, ba.a_off, ba.row_stride, ba.buf, ba.b_off, ba.row_stride,
                              dt, dt_bias, ssm_a, rows=T, hv=hv)
    want_out, want_state = oracle.prefill_varlen(
        cu_seqlens=cu, hk=hk, hv=hv, dk=dk, dv=dv, q=conv, q_off=0, q_rs=stride, k=conv,
        k_off=hk * dk, k_rs=stride, v=conv, v_off=2 * hk * dk, v_rs=stride, in_dt=dt, g=wg,
        beta=wb.astype(np.float32), pool=pool, idx=idx, has_init=None, scale=scale)
    got = H.out_to_f64(out)
    assert np.isfinite(got).all()
    assert H.rel_l1(got, want_out) <= H.OUT_TOL_HALF
    st = dpool[t(idx.astype(np.int64))].cpu().numpy()
    assert H.rel_l1(st, want_state) <= H.STATE_TOL


FUSED_CASES = [
    # (lengths, hk, hv, in dtype, a/b dtype, out dtype, rounded beta)
    ([70, 1, 1300, 64], 2, 4, W.BF16, W.BF16, W.BF16, True),
    ([33, 900], 1, 3, W.F16, W.F16, W.F32, False),
    ([200, 5, 17], 2, 2, W.BF16, W.F32, W.BF16, False),
]


@pytest.mark.parametrize("sequential", [True, False], ids=["sequential", "default"])
@pytest.mark.parametrize("spec", FUSED_CASES, ids=lambda s: "L{}-{}-ab{}-{}".format(
    "_".join(map(str, s[0])), W.DTYPE_NAMES[s[3]], W.DTYPE_NAMES[s[4]],
    "rounded" if s[6] else "f32beta"))
def test_prefill_with_the_gate_fused(dev, spec, sequential):
    """gdn_prefill_varlen_packed (q|k|v straight from padded conv rows, g and
    beta formed in the kernels from the raw b|a row) and
    gdn_prefill_varlen_gated (raw alpha, post-sigmoid beta) give the same bits
    as gdn_gate_beta / gdn_gate followed by gdn_prefill_varlen, and match the
    oracle."""
    lengths, hk, hv, dt, abd, outd, rounded = spec
    announce(f"prefill with the gate fused {spec} sequential={sequential}")
    dk, dv, pad = 128, 128, 8
    T = sum(lengths)
    rng = np.random.default_rng(5252 + T)
    width = 2 * hk * dk + hv * dv
    conv = W.nan_fill((T, width + pad), dt)
    conv[:, :width] = W.encode(rng.normal(size=(T, width)), dt)
    alpha, dt_bias, ssm_a = W.gate_inputs(rng, T, hv, large_every_third=True,
                                          head0_offset=0.0, a_log_hi=2.0)
    ba = W.merged_ba(5252 + T, alpha, abd)
    slots = len(lengths) + 2
    pool = W.make_pool(5252, slots, hv, dv, dk, 0.05)
    idx = rng.permutation(slots)[:len(lengths)].astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    scale = float(np.float32(1.0 / np.sqrt(dk)))
    t = lambda x: torch.from_numpy(x).to(dev)
    cd = H.to_dev(conv, dt, dev).reshape(-1)
    stride = width + pad
    q = cd.as_strided((T, hk, dk), (stride, dk, 1), 0)
    k = cd.as_strided((T, hk, dk), (stride, dk, 1), hk * dk)
    v = cd.as_strided((T, hv, dv), (stride, dv, 1), 2 * hk * dk)
    _, a, b = ba_views(ba, T, hv, dev)
    od = H.TORCH_OF[outd]
    kw = dict(scale=scale, state_idx=t(idx), sequential=sequential, out_dtype=od)
    # composed: materialised g and beta
    g, beta = gdn.gate_beta(a, b, t(dt_bias), t(ssm_a), rounded=rounded)
    pool_c = t(pool)
    out_c = gdn.prefill_varlen(q, k, v, g, beta, pool_c, t(cu), **kw)
    # packed: raw a and b
    pool_p = t(pool)
    out_p = gdn.prefill_varlen_packed(q, k, v, a, b, t(dt_bias), t(ssm_a), pool_p, t(cu),
                                      rounded=rounded, **kw)
    # gated: raw alpha (the a view) with the materialised post-sigmoid beta
    pool_g = t(pool)
    out_g = gdn.prefill_varlen_gated(q, k, v, a, t(dt_bias), t(ssm_a), beta, pool_g, t(cu),
                                     **kw)
    torch.cuda.synchronize()
    assert H.bytes_equal(out_p, out_c) and H.bytes_equal(pool_p, pool_c), "packed differs"
    assert H.bytes_equal(out_g, out_c) and H.bytes_equal(pool_g, pool_c), "gated differs"
    wg, wb = oracle.gate_beta(ba.buf, ba.a_off, ba.row_stride, ba.buf, ba.b_off, ba.row_stride,
                              abd, dt_bias, ssm_a, rows=T, hv=hv, round_beta=rounded)
    want_out, want_state = oracle.prefill_varlen(
        cu_seqlens=cu, hk=hk, hv=hv, dk=dk, dv=dv, q=conv, q_off=0, q_rs=stride, k=conv,
        k_off=hk * dk, k_rs=stride, v=conv, v_off=2 * hk * dk, v_rs=stride, in_dt=dt, g=wg,
        beta=wb.astype(np.float32), pool=pool, idx=idx, has_init=None, scale=scale)
    got = H.out_to_f64(out_p)
    assert np.isfinite(got).all()
    H.check_units(got, want_out, 2, H.tier_tol(dt, outd), "fused-gate prefill output")
    st = pool_p[t(idx.astype(np.int64))].cpu().numpy()
    H.check_units(st, want_state, 2, H.STATE_TOL, "fused-gate prefill state")
    assert H.bytes_equal(cd, H.to_dev(conv, dt, dev).reshape(-1)), "the conv rows were written"
