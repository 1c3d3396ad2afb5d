"""GPU tests of the slot table handling (vllm.cpp tests/vt/test_ops_gdn.cpp,
"gdn packed decode rejects duplicate and out-of-range live slots", and the
varlen cases' cu_seqlens = query_start_loc).

With GDN_CHECK_SLOTS the library reads the slot table (and cu_seqlens) back
and rejects a bad one before enqueueing anything: the pool and the output
keep their bytes.  Without it, a row or sequence whose slot is out of range
gets NaN outputs and no state access (the kernels' own bounds checks), and
every other row is computed as usual."""
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


def decode_inputs(case, dev):
    _, q, k, v = H.upload_views(case, dev, case.batch)
    t = lambda a: torch.from_numpy(a).to(dev)
    return q, k, v, t(case.alpha), t(case.dt_bias), t(case.ssm_a), t(case.beta), t(case.pool)


def small_decode():
    return W.make_decode_case("chk", 88, batch=5, hk=2, hv=4, dk=128, dv=64, in_dtype=W.BF16,
                              out_dtype=W.F32, slots=8, null_rows=(2,))


@pytest.mark.parametrize("bad", ["duplicate", "out_of_range"])
def test_decode_check_slots_rejects_and_enqueues_nothing(dev, bad):
    announce(f"decode GDN_CHECK_SLOTS: {bad}")
    case = small_decode()
    q, k, v, alpha, dt_bias, ssm_a, beta, pool = decode_inputs(case, dev)
    idx = case.idx.copy()
    if bad == "duplicate":
        idx[4] = idx[0]
    else:
        idx[3] = case.num_slots
    didx = torch.from_numpy(idx).to(dev)
    out = torch.full((case.batch, case.hv, case.dv), 7.0, device=dev)
    pool0 = pool.clone()
    with pytest.raises(gdn.GdnError) as ei:
        gdn.decode(q, k, v, alpha, dt_bias, ssm_a, beta, pool, didx, scale=case.scale,
                   out=out, check_slots=True)
    torch.cuda.synchronize()
    assert ei.value.code == -4, ei.value
    assert H.bytes_equal(pool, pool0)
    assert torch.all(out == 7.0)


def test_decode_check_slots_accepts_a_valid_table(dev):
    announce("decode GDN_CHECK_SLOTS: valid table with a padded row")
    case = small_decode()
    q, k, v, alpha, dt_bias, ssm_a, beta, pool = decode_inputs(case, dev)
    pool0 = pool.clone()
    out = gdn.decode(q, k, v, alpha, dt_bias, ssm_a, beta, pool,
                     torch.from_numpy(case.idx).to(dev), scale=case.scale,
                     out_dtype=torch.float32, check_slots=True)
    torch.cuda.synchronize()
    res = H.DecodeResult(H.out_to_f64(out), pool, pool0, True)
    want_out, want_state = oracle.decode_case(case)
    H.check_decode(case, res, want_out, want_state)


def test_decode_out_of_range_slot_unchecked_gives_nan_row(dev):
    announce("decode without the check: an out-of-range slot gives a NaN row, no state access")
    case = small_decode()
    q, k, v, alpha, dt_bias, ssm_a, beta, pool = decode_inputs(case, dev)
    idx = case.idx.copy()
    idx[3] = case.num_slots + 5
    pool0 = pool.clone()
    out = gdn.decode(q, k, v, alpha, dt_bias, ssm_a, beta, pool, torch.from_numpy(idx).to(dev),
                     scale=case.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = H.out_to_f64(out)
    assert np.isnan(got[3]).all()
    rows = [0, 1, 2, 4]
    want_out, want_state = oracle.decode_case(case, rows=rows)
    assert H.rel_l1(got[rows][[0, 1, 3]], want_out[[0, 1, 3]]) <= H.out_tol(case)
    assert np.all(got[2] == 0.0)
    live = [r for r in rows if case.idx[r] >= 0]
    touched = torch.from_numpy(case.idx[live].astype(np.int64)).to(dev)
    keep = np.setdiff1d(np.arange(case.num_slots), case.idx[live])
    keep_t = torch.from_numpy(keep).to(dev)
    assert H.bytes_equal(pool[keep_t], pool0[keep_t])
    got_state = pool[touched].cpu().numpy()
    want = want_state[[rows.index(r) for r in live]]
    assert H.rel_l1(got_state, want) <= H.STATE_TOL


def prefill_inputs(case, dev):
    _, q, k, v = H.upload_views(case, dev, case.total_tokens)
    t = lambda a: torch.from_numpy(a).to(dev)
    g = gdn.gate(t(case.alpha), t(case.dt_bias), t(case.ssm_a))
    return q, k, v, g, t(case.beta), t(case.pool)


def small_prefill():
    return W.make_prefill_case("chkp", 99, lengths=[70, 0, 5, 130], hk=2, hv=4, dk=128, dv=64,
                               in_dtype=W.BF16, out_dtype=W.BF16, slots=7,
                               has_init=[1, 1, 0, 1])


@pytest.mark.parametrize("sequential", [True, False], ids=["sequential", "default"])
@pytest.mark.parametrize("bad", ["duplicate", "negative", "out_of_range", "cu_end", "cu_down"])
def test_prefill_check_slots_rejects_and_enqueues_nothing(dev, bad, sequential):
    announce(f"prefill GDN_CHECK_SLOTS: {bad} sequential={sequential}")
    case = small_prefill()
    q, k, v, g, beta, pool = prefill_inputs(case, dev)
    idx, cu = case.idx.copy(), case.cu_seqlens.copy()
    code = -4
    if bad == "duplicate":
        idx[3] = idx[1]
    elif bad == "negative":
        idx[2] = -1
    elif bad == "out_of_range":
        idx[0] = case.num_slots
    elif bad == "cu_end":
        cu[-1] -= 1
        code = -3
    else:
        cu[2] = cu[1] - 1
        code = -3
    out = torch.full((case.total_tokens, case.hv, case.dv), 3.0, dtype=torch.bfloat16,
                     device=dev)
    pool0 = pool.clone()
    with pytest.raises(gdn.GdnError) as ei:
        gdn.prefill_varlen(q, k, v, g, beta, pool, torch.from_numpy(cu).to(dev),
                           scale=case.scale, state_idx=torch.from_numpy(idx).to(dev),
                           has_initial_state=torch.from_numpy(case.has_init).to(dev),
                           out=out, sequential=sequential, check_slots=True)
    torch.cuda.synchronize()
    assert ei.value.code == code, ei.value
    assert H.bytes_equal(pool, pool0)
    assert torch.all(out == 3.0)


@pytest.mark.parametrize("sequential", [True, False], ids=["sequential", "default"])
def test_prefill_check_slots_accepts_a_valid_table(dev, sequential):
    announce(f"prefill GDN_CHECK_SLOTS: valid table sequential={sequential}")
    case = small_prefill()
    q, k, v, g, beta, pool = prefill_inputs(case, dev)
    pool0 = pool.clone()
    out = gdn.prefill_varlen(q, k, v, g, beta, pool, torch.from_numpy(case.cu_seqlens).to(dev),
                             scale=case.scale, state_idx=torch.from_numpy(case.idx).to(dev),
                             has_initial_state=torch.from_numpy(case.has_init).to(dev),
                             out_dtype=torch.bfloat16, sequential=sequential,
                             check_slots=True)
    torch.cuda.synchronize()
    res = H.PrefillResult(H.out_to_f64(out), pool, pool0, True)
    want_out, want_state = oracle.prefill_case(case)
    H.check_prefill(case, res, want_out, want_state)


@pytest.mark.parametrize("aux", [False, True], ids=["one_stream", "split"])
def test_prefill_overlapping_cu_seqlens_stay_inside_the_workspace(dev, aux):
    """Without the check an overlapping cu_seqlens is clamped, not rejected.
    Here sequences 0 and 4 both cover all 6400 tokens: with the longest
    sequences ranked first, sequence 4's chunks are formed at record indices
    past the ceil(T / 64) + num_seqs records the workspace holds.  Nothing
    may be written past the workspace (a guard of 0xA5 bytes right behind it
    keeps its bytes), slots no sequence names keep theirs, empty sequences
    hand their states through, and sequence 0, whose records all fit, still
    ends in the oracle's state."""
    announce(f"prefill with overlapping cu_seqlens, unchecked, aux={aux}")
    case = W.make_prefill_case("ovl", 8800, lengths=[6400, 0, 0, 0, 0, 0], hk=2, hv=4,
                               dk=128, dv=128, in_dtype=W.BF16, out_dtype=W.BF16, slots=9,
                               has_init=[1] * 6)
    cu = np.array([0, 6400, 0, 64, 0, 6400, 6400], dtype=np.int32)
    q, k, v, g, beta, pool = prefill_inputs(case, dev)
    T, N = case.total_tokens, case.num_seqs
    ws_n = gdn.prefill_workspace_size(T, N, case.hk, case.hv, case.dk, case.dv, torch.bfloat16)
    guard = 1 << 18
    buf = torch.full((ws_n + guard,), 0xA5, dtype=torch.uint8, device=dev)
    pool0 = pool.clone()
    gdn.prefill_varlen(q, k, v, g, beta, pool, torch.from_numpy(cu).to(dev), scale=case.scale,
                       state_idx=torch.from_numpy(case.idx).to(dev),
                       has_initial_state=torch.from_numpy(case.has_init).to(dev),
                       out_dtype=torch.bfloat16, workspace=buf[:ws_n],
                       aux_stream=torch.cuda.Stream() if aux else None)
    torch.cuda.synchronize()
    assert torch.all(buf[ws_n:] == 0xA5), "bytes written past the workspace"
    idx = [int(x) for x in case.idx]
    for sl in range(case.num_slots):
        if sl not in idx or sl in (idx[1], idx[3], idx[5]):
            assert H.bytes_equal(pool[sl], pool0[sl]), f"slot {sl} changed"
    _, want_state = oracle.prefill_case(case)
    got = pool[idx[0]].float().cpu().numpy()[None]
    H.check_units(got, want_state[0:1], 2, H.STATE_TOL, "sequence 0 state")
