"""GPU parity of the gated RMSNorm (vllm.cpp tests/vt/test_ops_gdn.cpp,
"rmsnorm_gated: norm-then-gate, silu and sigmoid activations", the
CPU-vs-CUDA rmsnorm_gated cases and the rank-3 padded-row gate case): the
standalone kernel over a stored [T, Hv, Dv] output, the epilogue fused into
decode, and the prefill entry that runs the norm over its output in place.  Tolerances as for the recurrence (relative L1): 1e-5 for f32 data,
2e-2 for 16-bit outputs.  Gate rows are padded with NaN that must never be
read; padded decode rows are exact zeros."""
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


def z_view(norm, rows, hv, dv, dev):
    t = H.to_dev(norm.z.buf, norm.dtype, dev)
    return t.reshape(-1).as_strided((rows, hv, dv), (norm.z.row_stride, dv, 1), 0)


def tol(in_dt, out_dt):
    return H.tier_tol(in_dt, out_dt)


NORM_CASES = [
    # (T, hv, dv, dtype, out dtype, gate row padding, sigmoid)
    (37, 3, 128, W.BF16, W.BF16, 11, False),
    (37, 3, 128, W.BF16, W.F32, 0, True),
    (20, 2, 128, W.F32, W.F32, 8, False),
    (9, 4, 64, W.F16, W.F16, 4, True),
    (5, 2, 256, W.BF16, W.BF16, 0, False),
    (6, 3, 16, W.F32, W.F32, 0, True),
    (7, 2, 4, W.F16, W.F32, 0, False),         # dv < 8 halves: row kernel
    (7, 2, 8, W.F16, W.F32, 0, False),
    (11, 3, 48, W.BF16, W.BF16, 5, False),     # dv / 8 not a power of two: row kernel
    (4, 2, 130, W.F32, W.F32, 3, True),        # dv not a multiple of 4: row kernel
    (3, 1, 512, W.BF16, W.BF16, 0, False),
    (2, 2, 1024, W.BF16, W.F32, 8, True),      # dv / 8 = 128 > 64: row kernel
    (3, 2, 512, W.F32, W.F32, 0, False),       # dv / 4 = 128 > 64: row kernel
]


@pytest.mark.parametrize("spec", NORM_CASES, ids=lambda s: "T{}-hv{}-dv{}-{}-{}-pad{}-{}".format(
    s[0], s[1], s[2], W.DTYPE_NAMES[s[3]], W.DTYPE_NAMES[s[4]], s[5],
    "sigmoid" if s[6] else "silu"))
def test_rmsnorm_gated_matrix(dev, spec):
    T, hv, dv, dt, odt, pad, sig = spec
    announce(f"rmsnorm_gated {spec}")
    rng = np.random.default_rng(T * 1000 + dv)
    x = W.encode(rng.uniform(-6, 6, size=(T, hv, dv)), dt)
    norm = W.norm_inputs(T + dv, T, hv, dv, dt, pad=pad)
    xd = H.to_dev(x, dt, dev)
    x0 = xd.clone()
    zd = z_view(norm, T, hv, dv, dev)
    z0 = zd.clone()
    wd = H.to_dev(norm.w, dt, dev)
    out = gdn.rmsnorm_gated(xd, zd, wd, eps=norm.eps, sigmoid=sig, out_dtype=H.TORCH_OF[odt])
    torch.cuda.synchronize()
    got = H.out_to_f64(out)
    want = oracle.rmsnorm_gated(x, dt, norm.z.buf, dt, norm.z.row_stride, norm.w, dt, rows=T,
                                hv=hv, dv=dv, eps=norm.eps, sigmoid=sig)
    assert np.isfinite(got).all(), "a NaN gate pad was read"
    r = H.rel_l1(got, want)
    assert r <= tol(dt, odt), f"rel-L1 {r:.3e}"
    assert H.bytes_equal(xd, x0) and H.bytes_equal(zd, z0)


def test_rmsnorm_gated_prefill_size_sampled_rows(dev):
    """The launch the benchmark times: the [32768, 24, 128] fp16 prefill output
    (about 786k rows, thousands of workgroups) with an fp16 gate and weight;
    every output finite, 4096 sampled rows and the last one against the oracle."""
    T, hv, dv = 32768, 24, 128
    announce(f"rmsnorm_gated [{T}, {hv}, {dv}] fp16 sampled rows")
    gen = torch.Generator(device=dev)
    gen.manual_seed(4040)
    x = torch.randn((T, hv, dv), generator=gen, device=dev, dtype=torch.float32).to(torch.float16)
    norm = W.norm_inputs(404, T, hv, dv, W.F16)
    z = z_view(norm, T, hv, dv, dev)
    w = H.to_dev(norm.w, W.F16, dev)
    out = gdn.rmsnorm_gated(x, z, w, eps=norm.eps)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    rng = np.random.default_rng(4041)
    rows = np.concatenate([rng.choice(T * hv, size=4096, replace=False), [T * hv - 1]])
    ti, hi = rows // hv, rows % hv
    xs = x[torch.from_numpy(ti).to(dev), torch.from_numpy(hi).to(dev)].cpu().numpy()
    zs = norm.z.buf.reshape(T, -1)[ti[:, None], hi[:, None] * dv + np.arange(dv)]
    want = oracle.rmsnorm_gated(xs.reshape(-1, 1, dv), W.F16, np.ascontiguousarray(zs), W.F16, dv,
                                norm.w, W.F16, rows=rows.size, hv=1, dv=dv, eps=norm.eps)
    got = H.out_to_f64(out[torch.from_numpy(ti).to(dev), torch.from_numpy(hi).to(dev)])
    r = H.rel_l1(got, want.reshape(-1, dv))
    assert r <= H.OUT_TOL_HALF, f"rel-L1 {r:.3e}"


def test_rmsnorm_gated_hand_values(dev):
    announce("rmsnorm_gated: the pages' hand values")
    x = torch.tensor([[[3.0, 4.0]]], device=dev)
    z = torch.tensor([[[1.0, -1.0]]], device=dev)
    w = torch.tensor([2.0, 0.5], device=dev)
    silu = gdn.rmsnorm_gated(x, z, w, eps=0.0).cpu().numpy()[0, 0]
    sig = gdn.rmsnorm_gated(x, z, w, eps=0.0, sigmoid=True).cpu().numpy()[0, 0]
    np.testing.assert_allclose(silu, [1.2406475, -0.1521362], atol=1e-6)
    np.testing.assert_allclose(sig, [1.2406475, 0.1521362], atol=1e-6)


def run_decode_norm(case, norm, dev, *, sigmoid, pool=None, out_dtype=None):
    dbufs, q, k, v = H.upload_views(case, dev, case.batch)
    t = lambda a: torch.from_numpy(a).to(dev)
    alpha, dt_bias, ssm_a, beta, idx = (t(case.alpha), t(case.dt_bias), t(case.ssm_a),
                                        t(case.beta), t(case.idx))
    if pool is None:
        pool = t(case.pool)
    pool0 = pool.clone()
    z = z_view(norm, case.batch, case.hv, case.dv, dev)
    w = H.to_dev(norm.w, norm.dtype, dev)
    out = gdn.decode_gated_norm(q, k, v, alpha, dt_bias, ssm_a, beta, pool, idx, z, w,
                                scale=case.scale, norm_eps=norm.eps, sigmoid=sigmoid,
                                l2norm=case.l2norm, l2_eps=case.l2_eps,
                                out_dtype=out_dtype or H.TORCH_OF[case.out_dtype])
    torch.cuda.synchronize()
    return H.DecodeResult(H.out_to_f64(out), pool, pool0, True)


DECODE_NORM_CASES = [
    # (batch, hk, hv, dk, dv, in, out, slots, packed_pad, null_rows, gate pad, sigmoid)
    (5, 2, 4, 128, 128, W.BF16, W.BF16, 8, None, (1,), 13, False),
    (4, 1, 3, 128, 128, W.F32, W.F32, 5, None, (), 0, True),
    (6, 2, 4, 128, 72, W.F16, W.F16, 9, 64, (5,), 7, False),
    (3, 1, 2, 128, 256, W.BF16, W.F32, 4, None, (), 0, True),
    (4, 2, 4, 64, 200, W.BF16, W.BF16, 6, None, (0,), 0, False),
    (3, 1, 2, 256, 128, W.BF16, W.BF16, 4, None, (), 5, False),
    (4, 1, 2, 16, 16, W.F32, W.F32, 4, None, (), 0, False),
    (3, 1, 2, 32, 40, W.F16, W.F32, 4, None, (2,), 0, True),
    (2, 1, 1, 128, 256, W.BF16, W.BF16, 3, None, (), 0, False),   # 8 waves per head
    (2, 1, 2, 64, 500, W.F32, W.F32, 3, None, (), 0, True),
]


@pytest.mark.parametrize("spec", DECODE_NORM_CASES,
                         ids=lambda s: "B{}-hv{}-dk{}-dv{}-{}-{}-{}".format(
                             s[0], s[2], s[3], s[4], W.DTYPE_NAMES[s[5]], W.DTYPE_NAMES[s[6]],
                             "sigmoid" if s[11] else "silu"))
def test_decode_gated_norm_matrix(dev, spec):
    B, hk, hv, dk, dv, ind, outd, slots, pad, nulls, zpad, sig = spec
    announce(f"decode + gated norm {spec}")
    case = W.make_decode_case("dn", 3000 + B * dk + dv, batch=B, hk=hk, hv=hv, dk=dk, dv=dv,
                              in_dtype=ind, out_dtype=outd, slots=slots, packed_pad=pad,
                              null_rows=nulls, large_every_third=True)
    norm = W.norm_inputs(dv + B, B, hv, dv, ind, pad=zpad)
    res = run_decode_norm(case, norm, dev, sigmoid=sig)
    want_y, want_state = oracle.decode_norm_case(case, norm, sigmoid=sig)
    H.check_decode(case, res, want_y, want_state)


def test_decode_gated_norm_equals_decode_then_norm(dev):
    announce("fused decode norm vs gdn_decode then gdn_rmsnorm_gated (f32)")
    case = W.make_decode_case("dn2", 17, batch=6, hk=2, hv=4, dk=128, dv=128, in_dtype=W.F32,
                              out_dtype=W.F32, slots=8, null_rows=(3,))
    norm = W.norm_inputs(17, 6, 4, 128, W.F32, pad=9)
    fused = run_decode_norm(case, norm, dev, sigmoid=False)
    plain = H.run_decode(case, dev)
    z = z_view(norm, case.batch, case.hv, case.dv, dev)
    w = H.to_dev(norm.w, W.F32, dev)
    x = torch.from_numpy(plain.out.astype(np.float32)).to(dev)
    y = H.out_to_f64(gdn.rmsnorm_gated(x, z, w, eps=norm.eps))
    live = case.idx >= 0
    assert H.rel_l1(fused.out[live], y[live]) <= 1e-6
    assert np.all(fused.out[~live] == 0.0)
    # the same state update (the fused kernel's wider tile may round the
    # reductions in another order)
    idx = torch.from_numpy(case.idx[live].astype(np.int64)).to(dev)
    assert H.rel_l1(fused.pool[idx].cpu().numpy(), plain.pool[idx].cpu().numpy()) <= 1e-6


def test_decode_gated_norm_b256_sampled(dev):
    announce("decode + gated norm B=256 Hk16 Hv32 D128 bf16, bf16 pool: sampled rows")
    case = W.decode_b256()
    norm = W.norm_inputs(202, case.batch, case.hv, case.dv, W.BF16, pad=0)
    bits = H.pool_storage(case.pool, W.BF16)
    res = run_decode_norm(case, norm, dev, sigmoid=False, pool=H.to_dev(bits, W.BF16, dev))
    rows = np.unique(np.concatenate([np.random.default_rng(2).choice(256, 40, replace=False),
                                     [0, 255]]))
    want_y, want_state = oracle.decode_norm_case(case, norm, rows=rows, pool=bits,
                                                 state_dt=W.BF16)
    res.pool0 = None   # only sampled rows were computed by the oracle
    r_out, r_st = H.check_decode(case, res, want_y, want_state, rows=rows)
    print(f"  out rel-L1 {r_out:.3e}  state rel-L1 {r_st:.3e}", flush=True)


def test_decode_gated_norm_rejects_wide_heads(dev):
    announce("decode + gated norm: dv beyond one workgroup is rejected")
    case = W.make_decode_case("dnw", 5, batch=2, hk=1, hv=1, dk=256, dv=136, in_dtype=W.BF16,
                              out_dtype=W.BF16, slots=2)
    norm = W.norm_inputs(5, 2, 1, 136, W.BF16)
    with pytest.raises(gdn.GdnError) as ei:
        run_decode_norm(case, norm, dev, sigmoid=False)
    assert ei.value.code == -3


@pytest.mark.parametrize("sequential", [True, False], ids=["sequential", "default"])
def test_prefill_then_gated_norm(dev, sequential):
    announce(f"prefill then gated norm sequential={sequential}")
    case = W.make_prefill_case("pn", 4411, lengths=[130, 1, 64, 77], hk=2, hv=4, dk=128,
                               dv=128, in_dtype=W.BF16, out_dtype=W.BF16, slots=6,
                               has_init=[1, 0, 1, 1])
    norm = W.norm_inputs(4411, case.total_tokens, case.hv, case.dv, W.BF16, pad=6)
    res = H.run_prefill(case, dev, sequential=sequential)
    x = H.to_dev(W.encode(res.out, W.BF16), W.BF16, dev).view(case.total_tokens, case.hv,
                                                              case.dv)
    z = z_view(norm, case.total_tokens, case.hv, case.dv, dev)
    w = H.to_dev(norm.w, W.BF16, dev)
    y = H.out_to_f64(gdn.rmsnorm_gated(x, z, w, eps=norm.eps))
    want_y, _ = oracle.prefill_norm_case(case, norm)
    r = H.rel_l1(y, want_y)
    assert np.isfinite(y).all() and r <= H.OUT_TOL_HALF, f"rel-L1 {r:.3e}"


# ---------------------------------------------------------------------------
# the prefill entry with the gated norm (gdn_prefill_varlen_gated_norm): the
# gated prefill, then the norm in place over its output on the same stream
# ---------------------------------------------------------------------------
def run_prefill_norm(case, norm, dev, *, sigmoid, sequential=False, aux=False):
    dbufs, q, k, v = H.upload_views(case, dev, case.total_tokens)
    snap = [t.clone() for t in dbufs.values()]
    alpha, dt_bias, ssm_a, beta, cu, idx, has_init = (
        torch.from_numpy(x).to(dev) for x in (case.alpha, case.dt_bias, case.ssm_a, case.beta,
                                              case.cu_seqlens, case.idx, case.has_init))
    pool = torch.from_numpy(case.pool).to(dev)
    pool0 = pool.clone()
    z = z_view(norm, case.total_tokens, case.hv, case.dv, dev)
    w = H.to_dev(norm.w, norm.dtype, dev)
    zw = [z.clone(), w.clone()]
    y = gdn.prefill_varlen_gated_norm(q, k, v, alpha, dt_bias, ssm_a, beta, pool, cu, z, w,
                                      scale=case.scale, norm_eps=norm.eps, sigmoid=sigmoid,
                                      state_idx=idx, has_initial_state=has_init,
                                      l2norm=case.l2norm, l2_eps=case.l2_eps,
                                      sequential=sequential,
                                      aux_stream=torch.cuda.Stream() if aux else None)
    torch.cuda.synchronize()
    same = (all(H.bytes_equal(a, b) for a, b in zip(snap, dbufs.values())) and
            H.bytes_equal(zw[0], z) and H.bytes_equal(zw[1], w))
    return H.PrefillResult(H.out_to_f64(y), pool, pool0, same), y


# The elementwise bar of a normalised output.  y_i = o_i / rms(o) * w_i act(z_i)
# divides o's error, which is bounded relative to the row's scale (the
# per-unit bar of o), by the row's rms, so it reaches y as the same fraction
# of |w_i act(z_i)|; y's own rounding adds a fraction of |y_i|, and a 16-bit
# output has an absolute floor, the spacing of its subnormals (2^-24 for
# fp16; none that matters for bf16 or f32).  Hence
#   |y_got - y_want| <= c (|w_i act(z_i)| + |y_want|) + floor
# with c the per-unit relative-L1 bar of the output tier (1e-5 for f32 data,
# 2e-2 for a 16-bit output, whose o on rows of small rms sits about 1 % of
# the row's scale from the oracle's f64 o where large terms cancel).  An
# element that is wrong outright is off by about |y| or |w act(z)| and fails.
SUBNORMAL_FLOOR = {W.F32: 0.0, W.BF16: 0.0, W.F16: 2.0 ** -24}


def check_prefill_norm(case, res, want_y, want_state, norm, dev, sigmoid):
    name = f"{case.name} normalised output"
    assert np.isfinite(res.out).all(), f"{name}: non-finite"
    H.check_units(res.out, want_y, 2, H.out_tol(case), name)
    z = z_view(norm, case.total_tokens, case.hv, case.dv, dev).double().cpu().numpy()
    w = H.to_dev(norm.w, norm.dtype, dev).double().cpu().numpy()
    sg = 1.0 / (1.0 + np.exp(-z))
    gate = np.abs(w * (sg if sigmoid else z * sg))
    c = H.out_tol(case)
    floor = SUBNORMAL_FLOOR[case.out_dtype]
    ratio = (np.abs(res.out - want_y) - floor) / (gate + np.abs(want_y) + 1e-30)
    worst = float(ratio.max()) if ratio.size else 0.0
    print(f"  {name}: worst (|d| - {floor:g}) / (|w act(z)| + |y|) = {worst:.3e} (bar {c:g})",
          flush=True)
    bad = ratio > c
    assert not bad.any(), (f"{name}: {int(bad.sum())} elements outside {c:g} (|w act(z)| + |y|) "
                           f"+ {floor:g}, worst {worst:.3e}; first at {tuple(np.argwhere(bad)[0])}")
    # the states, the untouched slots and the inputs as for the plain prefill
    H.check_prefill(case, res, want_y, want_state, check_out=False)


PREFILL_NORM_CASES = [
    # (lengths, hk, hv, dk, dv, dtype, gate row padding, sigmoid, sequential)
    ([130, 1, 64, 77], 2, 4, 128, 128, W.BF16, 6, False, False),
    ([130, 1, 64, 77], 2, 4, 128, 128, W.BF16, 6, False, True),
    ([65, 200], 1, 3, 128, 64, W.F16, 0, True, False),
    ([40, 9], 2, 2, 64, 48, W.F32, 3, False, False),       # token-sequential; row norm kernel
    ([0, 33, 1], 1, 2, 32, 32, W.BF16, 0, True, False),    # an empty sequence
]


@pytest.mark.parametrize("spec", PREFILL_NORM_CASES,
                         ids=lambda s: "L{}-hv{}-dk{}-dv{}-{}-{}-{}".format(
                             "_".join(map(str, s[0])), s[2], s[3], s[4],
                             W.DTYPE_NAMES[s[5]], "sigmoid" if s[7] else "silu",
                             "sequential" if s[8] else "default"))
def test_prefill_gated_norm_matrix(dev, spec):
    lengths, hk, hv, dk, dv, dt, zpad, sig, seq = spec
    announce(f"prefill + gated norm {spec}")
    case = W.make_prefill_case("pgn", 5000 + sum(lengths) + dv, lengths=lengths, hk=hk, hv=hv,
                               dk=dk, dv=dv, in_dtype=dt, out_dtype=dt,
                               slots=len(lengths) + 2, has_init=[1, 0, 1, 1][:len(lengths)])
    norm = W.norm_inputs(5000 + dv, case.total_tokens, hv, dv, dt, pad=zpad)
    res, _ = run_prefill_norm(case, norm, dev, sigmoid=sig, sequential=seq)
    want_y, want_state = oracle.prefill_norm_case(case, norm, sigmoid=sig)
    check_prefill_norm(case, res, want_y, want_state, norm, dev, sig)


def test_prefill_gated_norm_equals_prefill_then_norm(dev):
    announce("prefill + gated norm vs gdn_prefill_varlen_gated then gdn_rmsnorm_gated, "
             "byte for byte (split schedule on a second stream)")
    case = W.make_prefill_case("pgn2", 77, lengths=[300, 129, 64, 5], hk=2, hv=4, dk=128,
                               dv=128, in_dtype=W.BF16, out_dtype=W.BF16, slots=6,
                               has_init=[1, 1, 0, 1])
    norm = W.norm_inputs(77, case.total_tokens, case.hv, case.dv, W.BF16, pad=5)
    _, y = run_prefill_norm(case, norm, dev, sigmoid=True, aux=True)
    dbufs, q, k, v = H.upload_views(case, dev, case.total_tokens)
    alpha, dt_bias, ssm_a, beta, cu, idx, has_init = (
        torch.from_numpy(x).to(dev) for x in (case.alpha, case.dt_bias, case.ssm_a, case.beta,
                                              case.cu_seqlens, case.idx, case.has_init))
    pool = torch.from_numpy(case.pool).to(dev)
    o = gdn.prefill_varlen_gated(q, k, v, alpha, dt_bias, ssm_a, beta, pool, cu,
                                 scale=case.scale, state_idx=idx, has_initial_state=has_init,
                                 l2norm=case.l2norm, l2_eps=case.l2_eps,
                                 aux_stream=torch.cuda.Stream())
    z = z_view(norm, case.total_tokens, case.hv, case.dv, dev)
    w = H.to_dev(norm.w, W.BF16, dev)
    y2 = gdn.rmsnorm_gated(o, z, w, eps=norm.eps, sigmoid=True)
    torch.cuda.synchronize()
    assert H.bytes_equal(y, y2)


def test_prefill_gated_norm_varlen_gqa3_all_heads(dev):
    announce("prefill + gated norm, varlen 8 seqs T=32768 Hk8 Hv24 GQA3 fp16: every head "
             "vs the oracle")
    case = W.prefill_varlen_gqa3()
    norm = W.norm_inputs(404, case.total_tokens, case.hv, case.dv, W.F16, pad=8)
    res, _ = run_prefill_norm(case, norm, dev, sigmoid=False, aux=True)
    want_y, want_state = oracle.prefill_norm_case(case, norm, sigmoid=False)
    check_prefill_norm(case, res, want_y, want_state, norm, dev, False)


def test_prefill_gated_norm_in_a_captured_graph(dev):
    """The entry's two launches captured into a graph (the whole call stays on
    the captured stream): every replay, from a restored pool, gives the eager
    call's normalised outputs and final states, and those match the oracle."""
    announce("prefill + gated norm captured into a graph: replays equal the eager call")
    case = W.make_prefill_case("pgng", 4545, lengths=[700, 130, 1, 64], hk=2, hv=4, dk=128,
                               dv=128, in_dtype=W.BF16, out_dtype=W.BF16, slots=6,
                               has_init=[1, 0, 1, 1])
    norm = W.norm_inputs(4545, case.total_tokens, case.hv, case.dv, W.BF16, pad=3)
    T, N = case.total_tokens, case.num_seqs
    _, q, k, v = H.upload_views(case, dev, T)
    t = lambda a: torch.from_numpy(a).to(dev)
    alpha, dt_bias, ssm_a, beta = t(case.alpha), t(case.dt_bias), t(case.ssm_a), t(case.beta)
    cu, idx, hi = t(case.cu_seqlens), t(case.idx), t(case.has_init)
    z = z_view(norm, T, case.hv, case.dv, dev)
    w = H.to_dev(norm.w, W.BF16, dev)
    pool0 = t(case.pool)
    ws = torch.empty(gdn.prefill_workspace_size(T, N, case.hk, case.hv, case.dk, case.dv,
                                                torch.bfloat16), dtype=torch.uint8, device=dev)
    out = torch.empty((T, case.hv, case.dv), dtype=torch.bfloat16, device=dev)
    pool = pool0.clone()

    def call():
        gdn.prefill_varlen_gated_norm(q, k, v, alpha, dt_bias, ssm_a, beta, pool, cu, z, w,
                                      scale=case.scale, norm_eps=norm.eps, sigmoid=True,
                                      state_idx=idx, has_initial_state=hi, out=out,
                                      workspace=ws, stream=torch.cuda.current_stream())

    call()
    torch.cuda.synchronize()
    want_out, want_pool = out.clone(), pool.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        pool.copy_(pool0)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            call()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        pool.copy_(pool0)
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_out), f"replay {rep}: outputs differ"
        assert H.bytes_equal(pool, want_pool), f"replay {rep}: states differ"
    want_y, want_s = oracle.prefill_norm_case(case, norm, sigmoid=True)
    check_prefill_norm(case, H.PrefillResult(H.out_to_f64(want_out), want_pool, pool0, True),
                       want_y, want_s, norm, dev, True)
