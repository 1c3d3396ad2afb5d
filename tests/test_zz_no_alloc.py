"""gdn_prefill_varlen_noalloc: the prefill entry point that allocates nothing
(its per-call records live in the library's fixed per-device scratch).
Called through the C ABI and compared with gdn_prefill_varlen (caller's
workspace) on the same inputs: outputs and final states bit-identical (the
same kernels run), and within the oracle's bars; two calls in a row, the
second smaller, so the second reads nothing the first left behind; a size
beyond the scratch is refused before anything is enqueued."""
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


def run_both(case, dev):
    """The case through gdn_prefill_varlen (own workspace) and through
    gdn_prefill_varlen_noalloc, each on its own copy of the pool."""
    _, q, k, v = H.upload_views(case, dev, case.total_tokens)
    t = lambda a: torch.from_numpy(a).to(dev)
    g = gdn.gate(t(case.alpha), t(case.dt_bias), t(case.ssm_a))
    beta, cu, idx, hi = t(case.beta), t(case.cu_seqlens), t(case.idx), t(case.has_init)
    pool0 = t(case.pool)
    od = H.TORCH_OF[case.out_dtype]
    pool_ws, pool_na = pool0.clone(), pool0.clone()
    out_ws = gdn.prefill_varlen(q, k, v, g, beta, pool_ws, cu, scale=case.scale, state_idx=idx,
                                has_initial_state=hi, out_dtype=od)
    out_na = torch.empty_like(out_ws)
    gdn.prefill_varlen_noalloc(q, k, v, g, beta, pool_na, cu, scale=case.scale, state_idx=idx,
                               has_initial_state=hi, out=out_na)
    torch.cuda.synchronize()
    return out_ws, pool_ws, out_na, pool_na, pool0


def check_case(case, dev):
    out_ws, pool_ws, out_na, pool_na, pool0 = run_both(case, dev)
    assert H.bytes_equal(out_na, out_ws), f"{case.name}: outputs differ from the workspace call"
    assert H.bytes_equal(pool_na, pool_ws), f"{case.name}: states differ from the workspace call"
    want_out, want_state = oracle.prefill_case(case)
    H.check_prefill(case, H.PrefillResult(H.out_to_f64(out_na), pool_na, pool0, True),
                    want_out, want_state, verbose=True)


def test_noalloc_two_calls_second_smaller(dev):
    announce("prefill noalloc: two calls, the second smaller, vs the workspace entry point")
    big = W.make_prefill_case("na-big", 8101, lengths=[700, 3, 1500, 0, 64], hk=2, hv=6,
                              dk=128, dv=128, in_dtype=W.BF16, out_dtype=W.BF16, slots=7,
                              has_init=[1, 1, 0, 1, 1])
    small = W.make_prefill_case("na-small", 8102, lengths=[130, 9], hk=1, hv=3, dk=128, dv=64,
                                in_dtype=W.F16, out_dtype=W.F32, slots=3, has_init=[0, 1])
    check_case(big, dev)
    check_case(small, dev)


def test_noalloc_t4096_then_small(dev):
    announce("prefill noalloc: one 4096-token sequence (Hk16 Hv32 bf16), then a small call")
    check_case(W.prefill_t4096(), dev)
    check_case(W.make_prefill_case("na-after", 8103, lengths=[65, 1], hk=2, hv=4, dk=128,
                                   dv=32, in_dtype=W.BF16, out_dtype=W.BF16, slots=2), dev)


def test_noalloc_refuses_sizes_beyond_the_scratch(dev):
    announce("prefill noalloc: a size beyond the scratch returns GDN_ERR_SHAPE, enqueues nothing")
    T, hk, hv, dk, dv = 32768, 2, 16, 128, 128
    need = gdn.prefill_workspace_size(T, 1, hk, hv, dk, dv, torch.bfloat16)
    assert need > gdn.gdn.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((T, hk, dk), dtype=torch.bfloat16, device=dev)
    v = torch.zeros((T, hv, dv), dtype=torch.bfloat16, device=dev)
    g = torch.zeros((T, hv), dtype=torch.float32, device=dev)
    pool = torch.full((1, hv, dv, dk), 3.0, dtype=torch.float32, device=dev)
    out = torch.full((T, hv, dv), 5.0, dtype=torch.bfloat16, device=dev)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    with pytest.raises(gdn.GdnError) as ei:
        gdn.prefill_varlen_noalloc(q, q, v, g, g, pool, cu, scale=0.088, out=out)
    assert ei.value.code == -3 and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((pool == 3.0).all()) and bool((out == 5.0).all())
