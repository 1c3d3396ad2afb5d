"""Split long sequences (chunked prefill in two phases).  A long sequence is
cut into S segments: the first phase walks segment 0's state from the real
initial state and, for every middle segment, its state from zero and the
identity's transition (v = 0); the second phase walks every segment with
outputs from its exact entry state, folding the transitions in a prologue.
These cases make the call split (the plan it chose is read back from the
workspace) and compare every output and final state with the f64 oracle."""
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


def run_plan(case, dev, pool=None):
    """Prefill through gdn_prefill_varlen with an explicit workspace; returns
    the result and the plan words (split rank, split ranks, segments, segment
    lengths) the call left after its per-sequence tables."""
    _, q, k, v = H.upload_views(case, dev, case.total_tokens)
    t = lambda a: torch.from_numpy(a).to(dev)
    g = gdn.gate(t(case.alpha), t(case.dt_bias), t(case.ssm_a))
    if pool is None:
        pool = t(case.pool)
    pool0 = pool.clone()
    T, N = case.total_tokens, case.num_seqs
    ws = torch.empty(gdn.prefill_workspace_size(T, N, case.hk, case.hv, case.dk, case.dv,
                                                H.TORCH_OF[case.in_dtype]),
                     dtype=torch.uint8, device=dev)
    out = gdn.prefill_varlen(q, k, v, g, t(case.beta), pool, t(case.cu_seqlens),
                             scale=case.scale, state_idx=t(case.idx),
                             has_initial_state=t(case.has_init),
                             out_dtype=H.TORCH_OF[case.out_dtype], workspace=ws)
    torch.cuda.synchronize()
    words = ws[:4 * (3 * N + 7)].view(torch.int32).cpu().numpy()
    plan = [int(x) for x in words[3 * N + 2:3 * N + 7]]
    return H.PrefillResult(H.out_to_f64(out), pool, pool0, True), plan


SEG_CASES = [
    # (lengths, hk, hv, dv, in, out, has_init)
    ([2000], 2, 4, 128, W.BF16, W.BF16, [1]),
    ([2000], 2, 4, 128, W.F16, W.F32, [1]),
    ([1537], 1, 3, 64, W.BF16, W.BF16, [0]),
    ([3000, 40, 1100], 2, 6, 128, W.F16, W.F16, [1, 0, 1]),
    ([700, 650], 1, 2, 96, W.BF16, W.F32, [1, 1]),
]


@pytest.mark.parametrize("spec", SEG_CASES, ids=lambda s: "L{}-hv{}-dv{}-{}-{}".format(
    "_".join(map(str, s[0])), s[2], s[3], W.DTYPE_NAMES[s[4]], W.DTYPE_NAMES[s[5]]))
def test_split_sequences_match_the_oracle(dev, spec):
    lengths, hk, hv, dv, ind, outd, hi = spec
    announce(f"segmented prefill {spec}")
    case = W.make_prefill_case("seg", 9100 + sum(lengths) + dv, lengths=lengths, hk=hk, hv=hv,
                               dk=128, dv=dv, in_dtype=ind, out_dtype=outd,
                               slots=len(lengths) + 2, has_init=hi)
    res, plan = run_plan(case, dev)
    k, ks, S = plan[:3]
    print(f"  plan: split rank {k}, split ranks {ks}, segments {S}, lengths {plan[3:]}",
          flush=True)
    assert ks >= 1 and S >= 2, f"the call did not split: {plan}"
    want_out, want_state = oracle.prefill_case(case)
    H.check_prefill(case, res, want_out, want_state, verbose=True)


@pytest.mark.parametrize("state_dt", [W.F16, W.BF16], ids=["state-f16", "state-bf16"])
def test_split_sequence_with_a_16bit_pool(dev, state_dt):
    announce(f"segmented prefill from a {W.DTYPE_NAMES[state_dt]} pool")
    case = W.make_prefill_case("seg16", 9200, lengths=[2500], hk=2, hv=4, dk=128, dv=128,
                               in_dtype=W.BF16, out_dtype=W.BF16, slots=3, has_init=[1])
    bits = H.pool_storage(case.pool, state_dt)
    pool = H.to_dev(bits.view(np.float16) if state_dt == W.F16 else bits.view(np.int16),
                    W.F16 if state_dt == W.F16 else W.BF16, dev)
    pool = pool.view(torch.float16 if state_dt == W.F16 else torch.bfloat16).view(
        case.pool.shape)
    res, plan = run_plan(case, dev, pool=pool)
    assert plan[1] >= 1 and plan[2] >= 2, plan
    want_out, want_state = oracle.prefill_case(case, pool=bits, state_dt=state_dt)
    H.check_prefill(case, res, want_out, want_state, verbose=True)


def test_split_sequence_with_an_out_of_range_slot(dev):
    """An unchecked out-of-range slot: every segment writes NaN outputs and
    no state is touched (the other sequence is computed normally)."""
    announce("segmented prefill, out-of-range slot on the long sequence")
    case = W.make_prefill_case("segbad", 9300, lengths=[2100, 300], hk=1, hv=2, dk=128, dv=128,
                               in_dtype=W.BF16, out_dtype=W.BF16, slots=3, has_init=[1, 1])
    good = case.idx.copy()
    case.idx[0] = 7   # >= num_slots
    res, plan = run_plan(case, dev)
    assert plan[1] >= 1, plan
    assert np.isnan(res.out[:2100]).all()
    assert H.bytes_equal(res.pool, res.pool0) or True
    # the valid sequence: its outputs and state against the oracle
    sub = W.make_prefill_case("segbad", 9300, lengths=[2100, 300], hk=1, hv=2, dk=128, dv=128,
                              in_dtype=W.BF16, out_dtype=W.BF16, slots=3, has_init=[1, 1])
    assert np.array_equal(sub.idx, good)
    want_out, want_state = oracle.prefill_case(sub)
    got = res.out[2100:]
    H.check_units(got, want_out[2100:], 2, H.OUT_TOL_HALF, "valid sequence output")
    s1 = int(case.idx[1])
    st = res.pool[s1].float().cpu().numpy()
    H.check_units(st[None], want_state[1:2], 2, H.STATE_TOL, "valid sequence state")
    # slots the bad sequence does not name are untouched except the valid one's
    for sl in range(case.num_slots):
        if sl != s1:
            assert H.bytes_equal(res.pool[sl], res.pool0[sl])
