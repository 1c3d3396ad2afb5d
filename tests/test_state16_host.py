"""CPU checks for the 16-bit state pool (vllm.cpp tests/vt/test_ops_gdn.cpp,
cases with FP16/BF16 persistent state): the oracle's reading of a stored
f16/bf16 pool, the checker the GPU tests apply to stored 16-bit states, and
the C ABI's validation of the state-format flags."""
import numpy as np
import pytest

import oracle
import workloads as W
import linear_attention_recurrence_gdn_amd as pkg
from tests import gpu_helpers as H
from tests.test_abi import _decode, _err, _prefill

SDTS = [W.F16, W.BF16]


def _widened(bits: np.ndarray, sdt: int) -> np.ndarray:
    # numpy's own half conversion and the bf16 bit shift: independent of the
    # oracle's decoders
    src = bits.view(np.float16) if sdt == W.F16 else bits
    return np.ascontiguousarray(W.decode_to_f32(src, sdt))


@pytest.mark.parametrize("sdt", SDTS, ids=["f16", "bf16"])
def test_decode_with_16bit_pool_equals_f32_pool_of_the_stored_values(sdt):
    case = W.make_decode_case("s16", 41, batch=3, hk=1, hv=2, dk=16, dv=8, in_dtype=W.F32,
                              out_dtype=W.F32, slots=5, null_rows=(1,))
    bits = H.pool_storage(case.pool, sdt)
    dec = _widened(bits, sdt)
    assert not np.array_equal(dec, case.pool)      # the encoding did round
    o16, s16 = oracle.decode_case(case, pool=bits, state_dt=sdt)
    o32, s32 = oracle.decode_case(case, pool=dec)
    np.testing.assert_array_equal(o16, o32)
    np.testing.assert_array_equal(s16, s32)


@pytest.mark.parametrize("sdt", SDTS, ids=["f16", "bf16"])
def test_prefill_with_16bit_pool_equals_f32_pool_of_the_stored_values(sdt):
    case = W.make_prefill_case("p16", 43, lengths=[5, 3, 0, 4], hk=1, hv=2, dk=16, dv=8,
                               in_dtype=W.F32, out_dtype=W.F32, slots=6,
                               has_init=[1, 0, 1, 1])
    bits = H.pool_storage(case.pool, sdt)
    dec = _widened(bits, sdt)
    o16, s16 = oracle.prefill_case(case, pool=bits, state_dt=sdt)
    o32, s32 = oracle.prefill_case(case, pool=dec)
    np.testing.assert_array_equal(o16, o32)
    np.testing.assert_array_equal(s16, s32)
    # the zero-length sequence hands its stored (widened) state through
    np.testing.assert_array_equal(s16[2], dec[case.idx[2]].astype(np.float64))
    # has_init == 0 never reads the (NaN) slot
    assert np.isfinite(s16[1]).all()


@pytest.mark.parametrize("sdt", SDTS, ids=["f16", "bf16"])
def test_rounded_state_checker_accepts_rne_and_rejects_one_ulp(sdt):
    rng = np.random.default_rng(7)
    want = rng.normal(0.0, 0.05, size=4096)
    want[:3] = [0.0, 1e-9, -3.0]
    bits = H.pool_storage(want.astype(np.float32), sdt)
    got = _widened(bits, sdt).astype(np.float64)
    H.check_state_rounded(got, want, sdt, "rne")
    bad = bits.copy()
    bad[100] ^= 1                                   # one ulp off in one element
    with pytest.raises(AssertionError):
        H.check_state_rounded(_widened(bad, sdt), want, sdt, "one-ulp")


def test_state_format_flags_are_validated():
    lib = pkg.load_library()
    both = 1 | (1 << 3) | (1 << 4)
    assert _decode(lib, flags=both) == -2 and "both set" in _err(lib)
    assert _prefill(lib, flags=both) == -2
    # a single state-format flag is accepted: the call reaches the null-pointer check
    for f in (1 << 3, 1 << 4):
        assert _decode(lib, flags=1 | f) == -1 and "null pointer" in _err(lib)
        assert _prefill(lib, flags=1 | f) == -1
