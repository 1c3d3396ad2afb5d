"""GPU parity of the depthwise causal conv1d (vllm.cpp tests/vt/test_ops_gdn.cpp:
the causal_conv1d_fwd / causal_conv1d_update cases, their CUDA varlen, indexed,
widened-cache and padded-row variants).  Outputs: relative L1 1e-5 for f32
data, 2e-2 for 16-bit outputs.  States are raw copies of inputs: every stored
state element must equal the oracle's value in the state format exactly.
Untouched slots, widened-cache tail columns and x padding keep their bytes."""
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


def tol(xd, od):
    return H.tier_tol(xd, od)


def stored(vals, sdt):
    """Oracle f64 values as the state format stores them (nearest even)."""
    enc = W.encode(vals, sdt)
    return W.decode_to_f32(enc, sdt).astype(np.float64)


def state_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def make_inputs(seed, T, C, K, xd, pad, slots, sl, sdt, with_bias):
    rng = np.random.default_rng(seed)
    x = W.nan_fill((max(T, 1), C + pad), xd)
    x[:T, :C] = W.encode(rng.normal(size=(T, C)), xd)
    w = W.encode(rng.uniform(-1, 1, size=(C, K)), xd)
    b = W.encode(rng.uniform(-1, 1, size=C), xd) if with_bias else None
    st = W.nan_fill((slots, C, max(sl, 1)), sdt)[:, :, :sl]
    st = np.ascontiguousarray(st)
    if K > 1:
        st[:, :, :K - 1] = W.encode(rng.normal(size=(slots, C, K - 1)), sdt)
    return x, w, b, st


FWD_CASES = [
    # (lengths, C, K, x dtype, out dtype, state dtype, bias, silu, has_init, indexed, x pad,
    #  extra state columns)
    ([5, 1, 3], 10, 4, W.F32, W.F32, W.F32, True, True, [1, 0, 1], False, 0, 0),
    ([1, 2], 3, 4, W.F32, W.F32, W.F32, False, False, [1, 0], False, 0, 0),
    ([9, 7], 512, 4, W.BF16, W.BF16, W.BF16, False, True, [1, 1], False, 0, 0),
    ([0, 17, 33, 1], 300, 3, W.F16, W.F32, W.F32, True, True, [1, 1, 0, 1], True, 8, 2),
    ([40], 64, 1, W.BF16, W.BF16, W.F32, True, False, [1], False, 0, 0),
    ([16, 16, 5], 96, 5, W.BF16, W.F32, W.F16, False, True, [0, 1, 1], True, 3, 1),
    ([70, 2, 130], 264, 8, W.F32, W.F32, W.BF16, True, True, [1, 1, 1], True, 0, 0),
    # 16-byte lanes with padded rows, zero-length and short sequences, a widened cache
    ([0, 3, 1, 20], 128, 4, W.BF16, W.BF16, W.BF16, True, True, [1, 0, 1, 1], True, 8, 1),
    ([9, 33], 64, 2, W.F16, W.F32, W.F16, False, False, [0, 1], False, 16, 0),
    # 16-byte lanes in 256- and 128-lane workgroups: sequences starting inside
    # 8-token spans and a partial last span
    ([37, 100, 5, 3], 2048, 4, W.BF16, W.BF16, W.BF16, True, True, [1, 0, 1, 1], True, 0, 0),
    ([25, 0, 41], 1024, 3, W.F16, W.F16, W.F32, False, True, [0, 1, 1], False, 0, 0),
]


@pytest.mark.parametrize("spec", FWD_CASES, ids=lambda s: "L{}-C{}-K{}-{}-{}-st{}".format(
    "_".join(map(str, s[0])), s[1], s[2], W.DTYPE_NAMES[s[3]], W.DTYPE_NAMES[s[4]],
    W.DTYPE_NAMES[s[5]]))
def test_conv1d_fwd_matrix(dev, spec):
    lengths, C, K, xd, od, sdt, bias, silu, hi, indexed, pad, extra = spec
    announce(f"conv1d_fwd {spec}")
    T, N = sum(lengths), len(lengths)
    slots = N + 3
    sl = K - 1 + extra
    x, w, b, st = make_inputs(31 * C + K, T, C, K, xd, pad, slots, sl, sdt, bias)
    rng = np.random.default_rng(C + K)
    idx = rng.permutation(slots)[:N].astype(np.int32) if indexed else None
    hi = np.asarray(hi, np.int8)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    t = lambda a: None if a is None else torch.from_numpy(a).to(dev)
    xd_t = H.to_dev(x, xd, dev)
    x0 = xd_t.clone()
    xv = xd_t.reshape(-1).as_strided((T, C), (C + pad, 1), 0)
    dstate = H.to_dev(st, sdt, dev) if K > 1 else None
    st0 = None if dstate is None else dstate.clone()
    out = gdn.conv1d_fwd(xv, H.to_dev(w, xd, dev), None if b is None else H.to_dev(b, xd, dev),
                         dstate, t(cu), state_idx=t(idx), has_initial_state=t(hi), silu=silu,
                         out_dtype=H.TORCH_OF[od])
    torch.cuda.synchronize()
    want, want_st = oracle.conv1d_fwd(cu_seqlens=cu, C=C, K=K, x=x, x_dt=xd, x_rs=C + pad, w=w,
                                      bias=b, state=st, st_dt=sdt, state_len=sl, idx=idx,
                                      has_init=hi, silu=silu)
    got = H.out_to_f64(out)
    assert np.isfinite(got).all()
    r = H.rel_l1(got, want)
    assert r <= tol(xd, od), f"rel-L1 {r:.3e}"
    assert H.bytes_equal(xd_t, x0)
    if K > 1:
        slots_used = idx if indexed else np.arange(N)
        gst = state_f64(dstate)
        np.testing.assert_array_equal(gst[slots_used][:, :, :K - 1], stored(want_st, sdt))
        untouched = np.setdiff1d(np.arange(slots), slots_used)
        ut = torch.from_numpy(untouched).to(dev)
        assert H.bytes_equal(dstate[ut], st0[ut])
        if extra:
            assert H.bytes_equal(dstate[:, :, K - 1:], st0[:, :, K - 1:])


@pytest.mark.parametrize("C,xd", [(256, W.BF16), (10, W.F32)], ids=["vec16B", "scalar"])
def test_conv1d_fwd_out_of_range_slot(dev, C, xd):
    """Unchecked slots: a sequence whose slot lies outside [0, num_slots) gets
    NaN in every output row (not only where its window would have been read)
    and keeps no state; its neighbours are unaffected."""
    announce(f"conv1d_fwd out-of-range slot C={C} {W.DTYPE_NAMES[xd]}")
    lengths, K = [20, 37, 11, 9], 4
    T, N, slots = sum(lengths), len(lengths), 6
    x, w, b, st = make_inputs(77 + C, T, C, K, xd, 0, slots, K - 1, W.F32, True)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    idx = np.asarray([4, slots + 5, 0, -1], np.int32)     # sequences 1 and 3 out of range
    hi = np.ones(N, np.int8)
    t = lambda a: torch.from_numpy(a).to(dev)
    dstate = H.to_dev(st, W.F32, dev)
    st0 = dstate.clone()
    out = gdn.conv1d_fwd(H.to_dev(x, xd, dev), H.to_dev(w, xd, dev), H.to_dev(b, xd, dev), dstate,
                         t(cu), state_idx=t(idx), has_initial_state=t(hi), out_dtype=torch.float32)
    torch.cuda.synchronize()
    # the oracle checks slots: give the two bad sequences valid slots there
    # (their neighbours' outputs and states do not depend on them)
    ok_idx = np.asarray([4, 1, 0, 2], np.int32)
    want, want_st = oracle.conv1d_fwd(cu_seqlens=cu, C=C, K=K, x=x, x_dt=xd, x_rs=C, w=w, bias=b,
                                      state=st, st_dt=W.F32, state_len=K - 1, idx=ok_idx,
                                      has_init=hi, silu=True)
    got = H.out_to_f64(out)
    for s in range(N):
        rows = slice(cu[s], cu[s + 1])
        if s in (1, 3):
            assert np.isnan(got[rows]).all(), f"sequence {s} not all NaN"
        else:
            assert H.rel_l1(got[rows], want[rows]) <= tol(xd, W.F32)
    gst = state_f64(dstate)
    np.testing.assert_array_equal(gst[[4, 0]], stored(want_st[[0, 2]], W.F32))
    ut = torch.tensor([1, 2, 3, 5], device=dev)
    assert H.bytes_equal(dstate[ut], st0[ut])


UPD_CASES = [
    # (batch, C, K, x dtype, out dtype, state dtype, bias, silu, indexed, x pad, extra)
    (4, 7, 4, W.F32, W.F32, W.F32, True, True, False, 0, 0),
    (3, 512, 4, W.BF16, W.BF16, W.BF16, False, True, True, 0, 0),
    (5, 100, 3, W.F16, W.F32, W.F32, True, False, True, 5, 1),
    (6, 256, 5, W.BF16, W.F32, W.F16, True, True, True, 0, 0),
    (2, 33, 1, W.F32, W.F32, W.F32, True, True, False, 0, 0),
    # 16-byte lanes: f32 / bf16 / f16 state rows of exactly K-1 entries, padded x rows,
    # a 64-lane workgroup at width 2, and the decode batch's shape
    (64, 1024, 4, W.F16, W.F16, W.F32, True, True, True, 8, 0),
    (7, 64, 2, W.BF16, W.BF16, W.F32, False, False, False, 0, 0),
    (256, 8192, 4, W.BF16, W.BF16, W.BF16, False, True, True, 0, 0),
    # a widened cache keeps the per-channel kernel
    (4, 512, 4, W.BF16, W.BF16, W.BF16, True, True, True, 0, 1),
]


@pytest.mark.parametrize("spec", UPD_CASES, ids=lambda s: "B{}-C{}-K{}-{}-{}-st{}".format(
    s[0], s[1], s[2], W.DTYPE_NAMES[s[3]], W.DTYPE_NAMES[s[4]], W.DTYPE_NAMES[s[5]]))
def test_conv1d_update_matrix(dev, spec):
    B, C, K, xd, od, sdt, bias, silu, indexed, pad, extra = spec
    announce(f"conv1d_update {spec}")
    slots = B + 2
    sl = K - 1 + extra
    x, w, b, st = make_inputs(17 * C + K, B, C, K, xd, pad, slots, sl, sdt, bias)
    if indexed:
        idx = (slots - 1 - np.arange(B)).astype(np.int32)
        idx[1] = -1                       # a padded row: output and state untouched
    else:
        idx = None
    t = lambda a: None if a is None else torch.from_numpy(a).to(dev)
    xv = H.to_dev(x, xd, dev).reshape(-1).as_strided((B, C), (C + pad, 1), 0)
    dstate = H.to_dev(st, sdt, dev) if K > 1 else None
    st0 = None if dstate is None else dstate.clone()
    out = torch.full((B, C), 5.0, dtype=H.TORCH_OF[od], device=dev)
    gdn.conv1d_update(xv, H.to_dev(w, xd, dev), None if b is None else H.to_dev(b, xd, dev),
                      dstate, state_idx=t(idx), silu=silu, out=out)
    torch.cuda.synchronize()
    want, want_st, written = oracle.conv1d_update(batch=B, C=C, K=K, x=x, x_dt=xd, x_rs=C + pad,
                                                  w=w, bias=b, state=st, st_dt=sdt,
                                                  state_len=sl, idx=idx, silu=silu)
    got = H.out_to_f64(out)
    assert np.all(got[~written] == 5.0)
    r = H.rel_l1(got[written], want[written])
    assert r <= tol(xd, od), f"rel-L1 {r:.3e}"
    if K > 1:
        rows = np.nonzero(written)[0]
        used = idx[rows] if indexed else rows
        gst = state_f64(dstate)
        np.testing.assert_array_equal(gst[used][:, :, :K - 1], stored(want_st[rows], sdt))
        untouched = torch.from_numpy(np.setdiff1d(np.arange(slots), used)).to(dev)
        assert H.bytes_equal(dstate[untouched], st0[untouched])
        if extra:
            assert H.bytes_equal(dstate[:, :, K - 1:], st0[:, :, K - 1:])


@pytest.mark.parametrize("C,xd", [(512, W.BF16), (36, W.F16)], ids=["vec16B", "scalar"])
def test_conv1d_update_out_of_range_slot(dev, C, xd):
    """Unchecked slots in the update: a row whose slot is past num_slots gets a
    NaN output row and touches no state; a negative slot leaves its output row
    and every state alone; the other rows match the oracle."""
    announce(f"conv1d_update out-of-range slot C={C} {W.DTYPE_NAMES[xd]}")
    B, K, slots = 5, 4, 6
    x, w, b, st = make_inputs(91 + C, B, C, K, xd, 0, slots, K - 1, W.BF16, True)
    idx = np.asarray([3, slots + 2, 0, -1, 5], np.int32)
    dstate = H.to_dev(st, W.BF16, dev)
    st0 = dstate.clone()
    out = torch.full((B, C), 5.0, dtype=torch.float32, device=dev)
    gdn.conv1d_update(H.to_dev(x, xd, dev), H.to_dev(w, xd, dev), H.to_dev(b, xd, dev), dstate,
                      state_idx=torch.from_numpy(idx).to(dev), out=out)
    torch.cuda.synchronize()
    ok_idx = np.asarray([3, 1, 0, -1, 5], np.int32)   # the oracle checks slots
    want, want_st, written = oracle.conv1d_update(batch=B, C=C, K=K, x=x, x_dt=xd, x_rs=C, w=w,
                                                  bias=b, state=st, st_dt=W.BF16,
                                                  state_len=K - 1, idx=ok_idx, silu=True)
    got = H.out_to_f64(out)
    assert np.isnan(got[1]).all()
    assert np.all(got[3] == 5.0)
    live = [0, 2, 4]
    assert H.rel_l1(got[live], want[live]) <= tol(xd, W.F32)
    gst = state_f64(dstate)
    np.testing.assert_array_equal(gst[[3, 0, 5]], stored(want_st[live], W.BF16))
    ut = torch.tensor([1, 2, 4], device=dev)
    assert H.bytes_equal(dstate[ut], st0[ut])


def test_conv1d_update_chain_equals_fwd(dev):
    announce("conv1d: update chain == fwd over the same tokens")
    T, C, K = 12, 130, 4
    x, w, b, st = make_inputs(99, T, C, K, W.F32, 0, 1, K - 1, W.F32, True)
    t = lambda a: torch.from_numpy(a).to(dev)
    s_fwd, s_upd = t(st), t(st)
    o_fwd = gdn.conv1d_fwd(t(x), t(w), t(b), s_fwd, t(np.array([0, T], np.int32)))
    outs = [gdn.conv1d_update(t(x[i:i + 1]), t(w), t(b), s_upd) for i in range(T)]
    torch.cuda.synchronize()
    o_upd = torch.cat(outs)
    assert H.rel_l1(o_upd.cpu().numpy(), o_fwd.cpu().numpy()) <= 1e-6
    assert torch.equal(s_fwd, s_upd)


def test_conv1d_fwd_varlen_workload_sampled_channels(dev):
    announce("conv1d_fwd over the 32768-token varlen workload, conv dim 5120 bf16: sampled")
    lengths = W.varlen_lengths(404)
    C, K = 2 * 8 * 128 + 24 * 128, 4
    T, N = sum(lengths), len(lengths)
    rng = np.random.default_rng(404)
    x = W.encode(rng.normal(size=(T, C)).astype(np.float32), W.BF16)
    w = W.encode(rng.uniform(-1, 1, size=(C, K)), W.BF16)
    st = W.encode(rng.normal(size=(64, C, K - 1)), W.BF16)
    idx = rng.permutation(64)[:N].astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    t = lambda a: torch.from_numpy(a).to(dev)
    dstate = H.to_dev(st, W.BF16, dev)
    out = gdn.conv1d_fwd(H.to_dev(x, W.BF16, dev), H.to_dev(w, W.BF16, dev), None, dstate, t(cu),
                         state_idx=t(idx))
    torch.cuda.synchronize()
    chans = np.sort(rng.choice(C, 48, replace=False))
    want, want_st = oracle.conv1d_fwd(cu_seqlens=cu, C=48, K=K, x=np.ascontiguousarray(x[:, chans]),
                                      x_dt=W.BF16, x_rs=48, w=np.ascontiguousarray(w[chans]),
                                      bias=None, state=np.ascontiguousarray(st[:, chans]),
                                      st_dt=W.BF16, state_len=K - 1, idx=idx, silu=True)
    got = H.out_to_f64(out)[:, chans]
    r = H.rel_l1(got, want)
    assert np.isfinite(got).all() and r <= H.OUT_TOL_HALF, f"rel-L1 {r:.3e}"
    gst = state_f64(dstate)[idx][:, chans]
    np.testing.assert_array_equal(gst, stored(want_st, W.BF16))
    print(f"  out rel-L1 {r:.3e}", flush=True)


def test_conv1d_check_slots(dev):
    announce("conv1d GDN_CHECK_SLOTS rejects duplicate slots and a bad cu_seqlens")
    T, C, K = 6, 8, 4
    x, w, b, st = make_inputs(5, T, C, K, W.F32, 0, 4, K - 1, W.F32, False)
    t = lambda a: torch.from_numpy(a).to(dev)
    dstate = t(st)
    s0 = dstate.clone()
    out = torch.full((T, C), 2.0, device=dev)
    with pytest.raises(gdn.GdnError) as ei:
        gdn.conv1d_fwd(t(x), t(w), None, dstate, t(np.array([0, 2, 6], np.int32)),
                       state_idx=t(np.array([1, 1], np.int32)), out=out, check_slots=True)
    assert ei.value.code == -4
    with pytest.raises(gdn.GdnError) as ei:
        gdn.conv1d_fwd(t(x), t(w), None, dstate, t(np.array([0, 4, 3], np.int32)), out=out,
                       check_slots=True)
    assert ei.value.code == -3
    torch.cuda.synchronize()
    assert torch.equal(dstate, s0) and torch.all(out == 2.0)
