"""GPU parity with the state pool stored as f16 or bf16 (vllm.cpp
tests/vt/test_ops_gdn.cpp, the packed-decode port and the CPU-vs-CUDA cases
with FP16/BF16 state: the stored state is widened to f32 for the step and the
new state rounded back on store).

The oracle reads the same stored 16-bit pool (widened exactly).  Outputs keep
the f32-state tolerances; each stored state element must be within half an
ulp of the oracle's f64 state (the one rounding on store) plus a small f32
allowance.  Padded rows are exact zeros; untouched slots and inputs keep their
bytes."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

STATE_DTS = [W.BF16, W.F16]
SDT_ID = lambda d: "state-" + W.DTYPE_NAMES[d]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def stored_pool(case, state_dt, dev):
    bits = H.pool_storage(case.pool, state_dt)
    return bits, H.to_dev(bits, state_dt, dev)


DECODE_CASES = [
    # (batch, hk, hv, dk, dv, in, out, slots, packed_pad, null_rows)
    (3, 1, 1, 16, 16, W.F32, W.F32, 4, None, ()),
    (4, 2, 4, 32, 40, W.BF16, W.BF16, 6, None, (0,)),
    (4, 1, 3, 64, 64, W.F16, W.F32, 5, None, (3,)),
    (7, 2, 6, 128, 128, W.BF16, W.BF16, 11, None, (2,)),
    (6, 2, 4, 128, 72, W.F16, W.F16, 9, 64, (5,)),
    (3, 1, 2, 256, 128, W.BF16, W.BF16, 4, None, ()),
]


@pytest.mark.parametrize("state_dt", STATE_DTS, ids=SDT_ID)
@pytest.mark.parametrize("spec", DECODE_CASES, ids=lambda s: "B{}-hk{}-hv{}-dk{}-dv{}-{}".format(
    s[0], s[1], s[2], s[3], s[4], W.DTYPE_NAMES[s[5]]))
def test_decode_state16(dev, spec, state_dt):
    B, hk, hv, dk, dv, ind, outd, slots, pad, nulls = spec
    announce(f"decode {W.DTYPE_NAMES[state_dt]} state {spec}")
    case = W.make_decode_case("d16", 6000 + B * dk + dv, batch=B, hk=hk, hv=hv, dk=dk, dv=dv,
                              in_dtype=ind, out_dtype=outd, slots=slots, packed_pad=pad,
                              null_rows=nulls, large_every_third=True)
    bits, pool = stored_pool(case, state_dt, dev)
    res = H.run_decode(case, dev, pool=pool)
    want_out, want_state = oracle.decode_case(case, pool=bits, state_dt=state_dt)
    H.check_decode(case, res, want_out, want_state)


@pytest.mark.parametrize("state_dt", STATE_DTS, ids=SDT_ID)
def test_decode_state16_beta0_g0_keeps_bits(dev, state_dt):
    announce(f"decode {W.DTYPE_NAMES[state_dt]} state: beta=0, g=0 keeps the stored bits")
    case = W.make_decode_case("d16inv", 9, batch=4, hk=2, hv=4, dk=128, dv=128,
                              in_dtype=W.BF16, out_dtype=W.F32, slots=6)
    case.beta[:] = 0.0
    case.ssm_a[:] = -0.0
    bits, pool = stored_pool(case, state_dt, dev)
    res = H.run_decode(case, dev, pool=pool)
    assert H.bytes_equal(res.pool, res.pool0)
    want_out, want_state = oracle.decode_case(case, pool=bits, state_dt=state_dt)
    H.check_decode(case, res, want_out, want_state, out_tolerance=1e-5)


@pytest.mark.parametrize("state_dt", STATE_DTS, ids=SDT_ID)
def test_decode_b256_state16_full(dev, state_dt):
    announce(f"decode B=256 Hk16 Hv32 D128 bf16, {W.DTYPE_NAMES[state_dt]} 1024-slot pool")
    case = W.decode_b256()
    bits, pool = stored_pool(case, state_dt, dev)
    res = H.run_decode(case, dev, pool=pool)
    want_out, want_state = oracle.decode_case(case, pool=bits, state_dt=state_dt)
    r_out, r_st = H.check_decode(case, res, want_out, want_state)
    print(f"  out rel-L1 {r_out:.3e}  state rel-L1 {r_st:.3e}", flush=True)


PREFILL_CASES = [
    # (lengths, hk, hv, dk, dv, in, out, has_init)
    ([1, 63, 64, 65, 130, 0], 2, 6, 128, 64, W.BF16, W.BF16, [1, 0, 1, 1, 0, 1]),
    ([200, 17], 1, 2, 128, 128, W.F16, W.F32, [1, 1]),
    ([33, 96], 1, 2, 64, 48, W.F32, W.F32, [1, 0]),
]


@pytest.mark.parametrize("sequential", [True, False], ids=["sequential", "default"])
@pytest.mark.parametrize("state_dt", STATE_DTS, ids=SDT_ID)
@pytest.mark.parametrize("spec", PREFILL_CASES, ids=lambda s: "L{}-dk{}-dv{}-{}".format(
    "_".join(map(str, s[0])), s[3], s[4], W.DTYPE_NAMES[s[5]]))
def test_prefill_state16(dev, spec, state_dt, sequential):
    lengths, hk, hv, dk, dv, ind, outd, hi = spec
    announce(f"prefill {W.DTYPE_NAMES[state_dt]} state {spec} sequential={sequential}")
    case = W.make_prefill_case("p16", 7000 + sum(lengths) + dv, lengths=lengths, hk=hk, hv=hv,
                               dk=dk, dv=dv, in_dtype=ind, out_dtype=outd,
                               slots=len(lengths) + 2, has_init=hi)
    bits, pool = stored_pool(case, state_dt, dev)
    res = H.run_prefill(case, dev, sequential=sequential, pool=pool)
    want_out, want_state = oracle.prefill_case(case, pool=bits, state_dt=state_dt)
    H.check_prefill(case, res, want_out, want_state)


@pytest.mark.parametrize("state_dt", STATE_DTS, ids=SDT_ID)
def test_prefill_varlen_gqa3_state16_all_heads(dev, state_dt):
    announce(f"prefill varlen 8 seqs T=32768 Hk8 Hv24 fp16, {W.DTYPE_NAMES[state_dt]} state, "
             f"every head")
    case = W.prefill_varlen_gqa3()
    bits, pool = stored_pool(case, state_dt, dev)
    res = H.run_prefill(case, dev, pool=pool)
    want_out, want_state = oracle.prefill_case(case, pool=bits, state_dt=state_dt)
    H.check_prefill(case, res, want_out, want_state, verbose=True)
