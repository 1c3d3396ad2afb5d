"""Host-side tests of the C ABI (no GPU): the library loads, exports every
entry point include/gdn.h declares, and rejects bad arguments before anything
is enqueued."""
import ctypes
import os
import re

import pytest
import torch

import linear_attention_recurrence_gdn_amd as pkg
from linear_attention_recurrence_gdn_amd import gdn as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gdn_gate", "gdn_decode", "gdn_prefill_varlen",
              "gdn_prefill_varlen_workspace_size", "gdn_last_error"):
        assert n in names, names


def test_library_exports_every_declared_symbol():
    lib = pkg.load_library()
    for n in declared_functions():
        assert hasattr(lib, n), n
    raw = ctypes.CDLL(B.LIB_PATH)
    for n in declared_functions():
        assert ctypes.cast(getattr(raw, n), ctypes.c_void_p).value


def test_binding_names_match_header():
    assert set(B.EXPORTS) == set(declared_functions())


# Argument checks.  Every device pointer is NULL or the checks fail before the
# null-pointer check, so nothing can be enqueued even on a machine with a GPU.
def _decode(lib, **kw):
    a = dict(out=None, out_dt=2, q=None, k=None, v=None, in_dt=2, q_rs=2048, k_rs=2048,
             v_rs=4096, alpha=None, alpha_dt=0, alpha_rs=32, dt_bias=None, ssm_a=None,
             beta=None, beta_rs=32, pool=None, slots=8, idx=None, batch=4, hk=16, hv=32,
             dk=128, dv=128, scale=0.088, eps=1e-6, flags=1, stream=None)
    a.update(kw)
    return lib.gdn_decode(*a.values())


def _err(lib):
    return lib.gdn_last_error().decode()


def test_decode_argument_errors():
    lib = pkg.load_library()
    assert _decode(lib, hv=33) == -3 and "multiple of Hk" in _err(lib)
    assert _decode(lib, dk=96) == -3 and "Dk = 96" in _err(lib)
    assert _decode(lib, scale=0.0) == -1 and "scale" in _err(lib)
    assert _decode(lib, scale=float("nan")) == -1
    assert _decode(lib, scale=float("inf")) == -1
    assert _decode(lib, eps=-1.0) == -1
    assert _decode(lib, in_dt=7) == -2
    assert _decode(lib, out_dt=1, in_dt=2) == -2      # f16 out from bf16 in
    assert _decode(lib, flags=1 << 9) == -1
    assert _decode(lib, batch=-1) == -3
    assert _decode(lib) == -1 and "null pointer" in _err(lib)
    assert _err(lib).startswith("gdn_decode:")
    # batch == 0 is a no-op
    assert _decode(lib, batch=0) == 0 and _err(lib) == ""


def _prefill(lib, **kw):
    a = dict(out=None, out_dt=1, q=None, k=None, v=None, in_dt=1, q_rs=1024, k_rs=1024,
             v_rs=3072, g=None, g_rs=24, beta=None, beta_rs=24, pool=None, slots=64,
             idx=None, has_init=None, cu=None, n=8, t=32768, hk=8, hv=24, dk=128, dv=128,
             scale=0.088, eps=1e-6, flags=1, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.gdn_prefill_varlen(*a.values())


def test_prefill_argument_errors():
    lib = pkg.load_library()
    assert _prefill(lib, hv=25) == -3
    assert _prefill(lib, scale=-1.0) == -1
    assert _prefill(lib, out_dt=2) == -2
    assert _prefill(lib, flags=1 << 5) == -1
    assert _prefill(lib) == -1 and _err(lib).startswith("gdn_prefill_varlen:")
    assert _prefill(lib, n=0) == 0


def _prefill_norm(lib, **kw):
    a = dict(out=None, out_dt=1, q=None, k=None, v=None, in_dt=1, q_rs=1024, k_rs=1024,
             v_rs=3072, alpha=None, alpha_dt=0, alpha_rs=24, dt_bias=None, ssm_a=None,
             beta=None, beta_rs=24, pool=None, slots=64, idx=None, has_init=None, cu=None,
             n=8, t=32768, hk=8, hv=24, dk=128, dv=128, scale=0.088, eps=1e-6, z=None,
             z_rs=3072, w=None, neps=1e-6, flags=1, ws=None, ws_bytes=0, stream=None, aux=None)
    a.update(kw)
    return lib.gdn_prefill_varlen_gated_norm(*a.values())


def test_prefill_gated_norm_argument_errors():
    # the norm's arguments are rejected before the prefill's own checks run
    lib = pkg.load_library()
    assert _prefill_norm(lib, out_dt=0) == -2 and "input dtype" in _err(lib)
    assert _prefill_norm(lib, neps=-1.0) == -1
    assert _prefill_norm(lib, neps=float("inf")) == -1
    assert _prefill_norm(lib, z_rs=3071) == -3 and "norm_z row stride" in _err(lib)
    assert _prefill_norm(lib) == -1 and "null pointer" in _err(lib)
    assert _err(lib).startswith("gdn_prefill_varlen_gated_norm:")
    # the sigmoid flag is the norm's, the prefill's checks never see it; a
    # prefill error is reported under this entry point's name
    assert _prefill_norm(lib, hv=25, z_rs=25 * 128) == -1     # the norm's null pointers first
    assert _prefill_norm(lib, t=0, hv=25) == -3 and "multiple of Hk" in _err(lib)
    assert _prefill_norm(lib, t=0, flags=1 | (1 << 5)) == -1 and "null pointer" in _err(lib)
    assert _prefill_norm(lib, t=0, flags=1 | (1 << 6)) == -1 and "unknown flags" in _err(lib)
    assert _prefill_norm(lib, n=0, t=0) == 0


def test_gate_argument_errors():
    lib = pkg.load_library()
    assert lib.gdn_gate(None, 32, None, 0, 32, None, None, 10, 0, None) == -3
    assert lib.gdn_gate(None, 16, None, 0, 32, None, None, 10, 32, None) == -3
    assert lib.gdn_gate(None, 32, None, 5, 32, None, None, 10, 32, None) == -2
    assert lib.gdn_gate(None, 32, None, 0, 32, None, None, 10, 32, None) == -1
    assert lib.gdn_gate(None, 32, None, 0, 32, None, None, 0, 32, None) == 0


@pytest.mark.skipif(torch.cuda.is_available(), reason="fake device pointers only without a GPU")
def test_alignment_and_stride_errors_without_gpu():
    lib = pkg.load_library()
    fake = 1 << 20   # never dereferenced: every call below fails validation
    kw = dict(out=fake, q=fake, k=fake, v=fake, alpha=fake, dt_bias=fake, ssm_a=fake,
              beta=fake, pool=fake, idx=fake)
    assert _decode(lib, **{**kw, "q": fake + 1}) == -1 and "aligned" in _err(lib)
    assert _decode(lib, **{**kw, "k_rs": 1024}) == -3
    assert _decode(lib, **{**kw, "v_rs": 100}) == -3
    assert _decode(lib, **{**kw, "pool": fake + 4}) == -1
    pk = dict(out=fake, q=fake, k=fake, v=fake, g=fake, beta=fake, pool=fake, cu=fake)
    assert _prefill(lib, **{**pk, "g_rs": 3}) == -3
    assert _prefill(lib, **pk, slots=4) == -4      # no state_idx and more seqs than slots


def test_binding_rejects_host_tensors():
    x = torch.zeros(4, 32)
    with pytest.raises(B.GdnError):
        pkg.gate(x, torch.zeros(32), torch.zeros(32))


def test_check_slots_flag_is_known():
    lib = pkg.load_library()
    # accepted by both entry points: validation goes on to the null-pointer check
    assert _decode(lib, flags=1 | (1 << 1)) == -1 and "null pointer" in _err(lib)
    assert _prefill(lib, flags=1 | (1 << 1)) == -1 and "null pointer" in _err(lib)
    assert B.GDN_CHECK_SLOTS == 1 << 1


def _norm(lib, **kw):
    a = dict(out=None, out_dt=2, x=None, x_dt=2, z=None, z_rs=3072, w=None, rows=16, hv=24,
             dv=128, eps=1e-6, flags=0, stream=None)
    a.update(kw)
    return lib.gdn_rmsnorm_gated(*a.values())


def test_rmsnorm_gated_argument_errors():
    lib = pkg.load_library()
    assert _norm(lib, x_dt=5) == -2
    assert _norm(lib, out_dt=1) == -2                   # f16 out from bf16 x
    assert _norm(lib, flags=1 << 6) == -1
    assert _norm(lib, flags=1) == -1                    # not a norm flag
    assert _norm(lib, eps=-1.0) == -1
    assert _norm(lib, eps=float("nan")) == -1
    assert _norm(lib, z_rs=3071) == -3
    assert _norm(lib, hv=0) == -3
    assert _norm(lib, flags=1 << 5) == -1 and "null pointer" in _err(lib)
    assert _err(lib).startswith("gdn_rmsnorm_gated:")
    assert _norm(lib, rows=0) == 0


def _decode_norm(lib, **kw):
    a = dict(out=None, out_dt=2, q=None, k=None, v=None, in_dt=2, q_rs=2048, k_rs=2048,
             v_rs=4096, alpha=None, alpha_dt=0, alpha_rs=32, dt_bias=None, ssm_a=None,
             beta=None, beta_rs=32, pool=None, slots=8, idx=None, batch=4, hk=16, hv=32,
             dk=128, dv=128, scale=0.088, eps=1e-6, z=None, z_rs=4096, w=None, neps=1e-6,
             flags=1, stream=None)
    a.update(kw)
    return lib.gdn_decode_gated_norm(*a.values())


def test_decode_gated_norm_argument_errors():
    lib = pkg.load_library()
    assert _decode_norm(lib, dk=256, dv=136) == -3 and "dv <= 128" in _err(lib)
    assert _decode_norm(lib, dk=128, dv=264) == -3 and "dv <= 256" in _err(lib)
    assert _decode_norm(lib, dk=64, dv=520) == -3 and "dv <= 512" in _err(lib)
    assert _decode_norm(lib, neps=-1.0) == -1
    assert _decode_norm(lib, flags=1 | (1 << 6)) == -1
    # the sigmoid flag belongs to the norm entry points only
    assert _decode(lib, flags=1 | (1 << 5)) == -1 and "unknown flags" in _err(lib)
    assert _decode_norm(lib, flags=1 | (1 << 5)) == -1 and "null pointer" in _err(lib)
    assert _err(lib).startswith("gdn_decode_gated_norm:")
    assert _decode_norm(lib, batch=0) == 0


def test_gate_beta_and_post_conv_argument_errors():
    lib = pkg.load_library()
    gb = lambda **kw: lib.gdn_gate_beta(*dict(dict(
        g=None, beta=None, out_rs=24, a=None, b=None, ab_dt=2, a_rs=48, b_rs=48, dt_bias=None,
        ssm_a=None, rows=8, hv=24, flags=0, stream=None), **kw).values())
    assert gb(ab_dt=7) == -2
    assert gb(flags=1 << 6) == -1                  # the decode-only raw-beta flag
    assert gb(out_rs=23) == -3 and gb(a_rs=23) == -3 and gb(b_rs=23) == -3
    assert gb(flags=1 << 7) == -1 and "null pointer" in _err(lib)
    assert _err(lib).startswith("gdn_gate_beta:")
    assert gb(rows=0) == 0
    pc = lambda **kw: lib.gdn_post_conv(*dict(dict(
        q=None, k=None, v=None, out_dt=2, g=None, beta=None, conv=None, conv_dt=2,
        conv_rs=8192, a=None, b=None, ab_dt=2, a_rs=64, b_rs=64, dt_bias=None, ssm_a=None,
        t=16, hk=16, hv=32, dk=128, dv=128, eps=1e-6, flags=0, stream=None), **kw).values())
    assert pc(conv_rs=8191) == -3
    assert pc(hv=33) == -3
    assert pc(conv_dt=9) == -2
    assert pc(eps=-1.0) == -1
    assert pc(flags=1) == -1
    assert pc() == -1 and "null pointer" in _err(lib)
    assert _err(lib).startswith("gdn_post_conv:")
    assert pc(t=0) == 0


def test_conv1d_argument_errors():
    lib = pkg.load_library()
    cf = lambda **kw: lib.gdn_conv1d_fwd(*dict(dict(
        out=None, out_dt=2, x=None, x_dt=2, x_rs=5120, w=None, b=None, st=None, sl=3, slots=64,
        idx=None, hi=None, cu=None, n=8, t=32768, c=5120, k=4, flags=1 << 8,
        stream=None), **kw).values())
    assert cf(k=9) == -3 and "width" in _err(lib)
    assert cf(k=0) == -3
    assert cf(sl=2) == -3 and "state_len" in _err(lib)
    assert cf(x_rs=5119) == -3
    assert cf(out_dt=1) == -2
    assert cf(flags=(1 << 3) | (1 << 4)) == -2
    assert cf(flags=1) == -1                       # not a conv flag
    assert cf(n=65, slots=64) == -4                # more sequences than slots, no index
    assert cf() == -1 and "null pointer" in _err(lib)
    assert _err(lib).startswith("gdn_conv1d_fwd:")
    assert cf(n=0) == 0
    cu = lambda **kw: lib.gdn_conv1d_update(*dict(dict(
        out=None, out_dt=2, x=None, x_dt=2, x_rs=8192, w=None, b=None, st=None, sl=3,
        slots=1024, idx=None, batch=256, c=8192, k=4, flags=1 << 8, stream=None), **kw).values())
    assert cu(k=9) == -3 and cu(sl=1) == -3
    assert cu(batch=2048) == -4
    assert cu(batch=2048, k=1) == -1 and "null pointer" in _err(lib)   # width 1: no state
    assert cu() == -1 and _err(lib).startswith("gdn_conv1d_update:")
    assert cu(batch=0) == 0


def test_prefill_noalloc_refuses_sizes_beyond_its_scratch():
    """The allocation-free prefill checks its fixed scratch against the call's
    sizes before anything else (host only: nothing is enqueued)."""
    lib = pkg.load_library()
    T, hk, hv, dk, dv = 32768, 2, 16, 128, 128
    assert lib.gdn_prefill_varlen_workspace_size(T, 1, hk, hv, dk, dv, 2, 1) > B.NOALLOC_SCRATCH_BYTES
    rc = lib.gdn_prefill_varlen_noalloc(None, 2, None, None, None, 2, hk * dk, hk * dk, hv * dv,
                                        None, hv, None, hv, None, 1, None, None, None, 1, T, hk,
                                        hv, dk, dv, 0.088, 1e-6, 1, None)
    assert rc == -3 and "scratch" in _err(lib)
    assert _err(lib).startswith("gdn_prefill_varlen_noalloc:")


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define GDN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.NOALLOC_SCRATCH_BYTES
