"""CPU oracle for the Gated DeltaNet hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
loads it.  The arithmetic lives in ``gdn_oracle.c`` (plain C, double precision);
this module compiles it with gcc and marshals numpy arrays through ctypes.

Parity status of every function: pinned (see tests/test_oracle_pins.py).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, F16, BF16 = 0, 1, 2
F64 = 3   # oracle-internal code: an array of doubles (e.g. an oracle output)


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c -> liboracle.so (gcc -O2, strict IEEE: no fast-math,
    no FMA contraction, so every product and sum is rounded as written)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=gnu99", "-pthread", "-fPIC", "-shared",
                               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, vp, dbl, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
        lib.oracle_decode_value.restype = dbl
        lib.oracle_decode_value.argtypes = [vp, i32, i64]
        lib.oracle_softplus.restype = None
        lib.oracle_softplus.argtypes = [vp, vp, i64]
        lib.oracle_gate.restype = i32
        lib.oracle_gate.argtypes = [i64, i64, vp, i32, i64, vp, vp, vp]
        lib.oracle_l2norm.restype = None
        lib.oracle_l2norm.argtypes = [vp, vp, i64, i64, dbl]
        lib.oracle_decode.restype = i32
        lib.oracle_decode.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, i32, i64, i64, i64,
                                      vp, vp, i64, vp, i32, i64, vp, dbl, dbl, i32, vp, vp,
                                      vp]
        lib.oracle_prefill_varlen.restype = i32
        lib.oracle_prefill_varlen.argtypes = [i64, vp, i64, i64, i64, i64, vp, vp, vp, i32,
                                              i64, i64, i64, vp, vp, i64, vp, i32, i64, vp,
                                              vp, dbl, dbl, i32, vp, vp, vp]
        lib.oracle_round_through.restype = dbl
        lib.oracle_round_through.argtypes = [ctypes.c_float, i32]
        lib.oracle_gate_beta.restype = i32
        lib.oracle_gate_beta.argtypes = [i64, i64, vp, vp, i32, i64, i64, vp, vp, i32, vp, vp]
        lib.oracle_post_conv.restype = i32
        lib.oracle_post_conv.argtypes = [i64, i64, i64, i64, i64, vp, i32, i64, vp, vp, i32,
                                         i64, i64, vp, vp, dbl, vp, vp, vp, vp, vp]
        lib.oracle_conv1d_fwd.restype = i32
        lib.oracle_conv1d_fwd.argtypes = [i64, vp, i64, i64, vp, i32, i64, vp, vp, vp, i32, i64,
                                          i64, vp, vp, i32, vp, vp]
        lib.oracle_conv1d_update.restype = i32
        lib.oracle_conv1d_update.argtypes = [i64, i64, i64, vp, i32, i64, vp, vp, vp, i32, i64,
                                             i64, vp, i32, vp, vp, vp]
        lib.oracle_rmsnorm_gated.restype = i32
        lib.oracle_rmsnorm_gated.argtypes = [i64, i64, i64, vp, i32, vp, i32, i64, vp, i32,
                                             dbl, i32, vp]
        lib.oracle_set_threads.restype = None
        lib.oracle_set_threads.argtypes = [i32]
        lib.oracle_get_threads.restype = i32
        lib.oracle_get_threads.argtypes = []
        lib.oracle_set_threads(default_threads())
        _lib = lib
    return _lib


def default_threads() -> int:
    """Host threads for the (row or sequence, v-head) units of decode and
    prefill: the CPUs this process may run on, at most 16 (one GPU's share of
    a host), or ORACLE_THREADS when set."""
    env = os.environ.get("ORACLE_THREADS")
    if env:
        return max(1, int(env))
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def set_threads(n: int) -> None:
    """Threads for decode and prefill units (the arithmetic of a unit does not
    depend on it)."""
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


class OracleError(RuntimeError):
    pass


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _need(a: np.ndarray, dtype) -> np.ndarray:
    assert a.dtype == dtype and a.flags.c_contiguous, (a.dtype, dtype)
    return a


def _pool(pool: np.ndarray, state_dt: int) -> np.ndarray:
    """The state pool as stored: float32 for F32, raw uint16 bits for F16/BF16."""
    if state_dt == F32:
        return _need(pool, np.float32)
    assert state_dt in (F16, BF16), state_dt
    return _need(pool, np.uint16)


def decode_value(buf: np.ndarray, dt: int, off: int) -> float:
    return _load().oracle_decode_value(_p(buf), dt, off)


def softplus(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    _load().oracle_softplus(_p(x), _p(y), x.size)
    return y


def l2norm(x, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    d = x.shape[-1]
    y = np.empty_like(x)
    _load().oracle_l2norm(_p(x), _p(y), x.size // d, d, float(eps))
    return y


def gate(alpha: np.ndarray, alpha_dt: int, dt_bias: np.ndarray, ssm_a: np.ndarray,
         alpha_row_stride: Optional[int] = None) -> np.ndarray:
    """g [rows, hv] f64 from alpha [rows, hv] (storage array, 2-D)."""
    rows = alpha.shape[0]
    hv = dt_bias.shape[0]
    rs = alpha.shape[1] if alpha_row_stride is None else alpha_row_stride
    g = np.empty((rows, hv), dtype=np.float64)
    rc = _load().oracle_gate(rows, hv, _p(np.ascontiguousarray(alpha)), alpha_dt, rs,
                             _p(_need(dt_bias, np.float32)), _p(_need(ssm_a, np.float32)),
                             _p(g))
    if rc:
        raise OracleError(f"oracle_gate: error {rc}")
    return g


def decode(*, batch, hk, hv, dk, dv, q, q_off, q_rs, k, k_off, k_rs, v, v_off, v_rs, in_dt,
           g, beta, pool, idx, scale, l2_eps=1e-6, l2norm=True, head_mask=None,
           state_out=None, state_dt=F32):
    """One decode step.  q/k/v are storage buffers addressed as
    buf.flat[off + row*rs + head*D + d].  The pool [slots,hv,dv,dk] is stored
    as state_dt (float32, or uint16 bits of f16/bf16).  Returns (out [B,hv,dv]
    f64, state_out [B,hv,dv,dk] f64 = updated states of the live rows)."""
    lib = _load()
    g = np.ascontiguousarray(g, dtype=np.float64)
    beta = _need(beta, np.float32)
    pool = _pool(pool, state_dt)
    idx = _need(np.asarray(idx, dtype=np.int32), np.int32)
    out = np.zeros((batch, hv, dv), dtype=np.float64)
    if state_out is None:
        state_out = np.zeros((batch, hv, dv, dk), dtype=np.float64)
    hm = None if head_mask is None else np.ascontiguousarray(head_mask, dtype=np.uint8)
    es = q.itemsize
    rc = lib.oracle_decode(batch, hk, hv, dk, dv,
                           q.ctypes.data + q_off * es, k.ctypes.data + k_off * es,
                           v.ctypes.data + v_off * es, in_dt, q_rs, k_rs, v_rs,
                           _p(g), _p(beta), beta.shape[1], _p(pool), int(state_dt),
                           pool.shape[0], _p(idx),
                           float(scale), float(l2_eps), int(bool(l2norm)), _p(hm),
                           _p(out), _p(state_out))
    if rc:
        raise OracleError(f"oracle_decode: error {rc}")
    return out, state_out


def prefill_varlen(*, cu_seqlens, hk, hv, dk, dv, q, q_off, q_rs, k, k_off, k_rs, v, v_off,
                   v_rs, in_dt, g, beta, pool, idx, has_init, scale, l2_eps=1e-6,
                   l2norm=True, head_mask=None, state_dt=F32):
    """Varlen prefill.  The pool is stored as state_dt (as for decode).
    Returns (out [T,hv,dv] f64, final states [N,hv,dv,dk] f64)."""
    lib = _load()
    cu = _need(np.asarray(cu_seqlens, dtype=np.int32), np.int32)
    n = cu.shape[0] - 1
    t = int(cu[-1])
    g = np.ascontiguousarray(g, dtype=np.float64)
    beta = _need(beta, np.float32)
    pool = _pool(pool, state_dt)
    idx_a = None if idx is None else _need(np.asarray(idx, dtype=np.int32), np.int32)
    hi = None if has_init is None else _need(np.asarray(has_init, dtype=np.int8), np.int8)
    hm = None if head_mask is None else np.ascontiguousarray(head_mask, dtype=np.uint8)
    out = np.zeros((t, hv, dv), dtype=np.float64)
    st = np.zeros((n, hv, dv, dk), dtype=np.float64)
    es = q.itemsize
    rc = lib.oracle_prefill_varlen(n, _p(cu), hk, hv, dk, dv,
                                   q.ctypes.data + q_off * es, k.ctypes.data + k_off * es,
                                   v.ctypes.data + v_off * es, in_dt, q_rs, k_rs, v_rs,
                                   _p(g), _p(beta), beta.shape[1], _p(pool), int(state_dt),
                                   pool.shape[0],
                                   _p(idx_a), _p(hi), float(scale), float(l2_eps),
                                   int(bool(l2norm)), _p(hm), _p(out), _p(st))
    if rc:
        raise OracleError(f"oracle_prefill_varlen: error {rc}")
    return out, st


def round_through(x: float, dt: int) -> float:
    return _load().oracle_round_through(float(x), dt)


def gate_beta(a_buf, a_off, a_rs, b_buf, b_off, b_rs, ab_dt, dt_bias, ssm_a, *, rows, hv,
              round_beta=False):
    """g and beta [rows, hv] f64 from raw a and b read as buf.flat[off + r*rs + h]
    (views of one merged row allowed).  round_beta: beta rounded through the
    storage dtype (the packed decode's rule)."""
    lib = _load()
    g = np.empty((rows, hv), dtype=np.float64)
    beta = np.empty((rows, hv), dtype=np.float64)
    ea, eb = a_buf.itemsize, b_buf.itemsize
    rc = lib.oracle_gate_beta(rows, hv, a_buf.ctypes.data + a_off * ea,
                              b_buf.ctypes.data + b_off * eb, ab_dt, a_rs, b_rs,
                              _p(_need(dt_bias, np.float32)), _p(_need(ssm_a, np.float32)),
                              int(bool(round_beta)), _p(g), _p(beta))
    if rc:
        raise OracleError(f"oracle_gate_beta: error {rc}")
    return g, beta


def post_conv(conv, conv_dt, conv_rs, a_buf, a_off, a_rs, b_buf, b_off, b_rs, ab_dt, dt_bias,
              ssm_a, *, T, hk, hv, dk, dv, l2_eps=1e-6):
    """The post-conv front-end: (q, k normalised [T,hk,dk], v [T,hv,dv], g, beta
    [T,hv]), all f64."""
    lib = _load()
    conv = np.ascontiguousarray(conv)
    q = np.empty((T, hk, dk)); k = np.empty((T, hk, dk)); v = np.empty((T, hv, dv))
    g = np.empty((T, hv)); beta = np.empty((T, hv))
    ea, eb = a_buf.itemsize, b_buf.itemsize
    rc = lib.oracle_post_conv(T, hk, hv, dk, dv, _p(conv), conv_dt, conv_rs,
                              a_buf.ctypes.data + a_off * ea, b_buf.ctypes.data + b_off * eb,
                              ab_dt, a_rs, b_rs, _p(_need(dt_bias, np.float32)),
                              _p(_need(ssm_a, np.float32)), float(l2_eps), _p(q), _p(k), _p(v),
                              _p(g), _p(beta))
    if rc:
        raise OracleError(f"oracle_post_conv: error {rc}")
    return q, k, v, g, beta


def rmsnorm_gated(x, x_dt, z, z_dt, z_row_stride, w, w_dt, *, rows, hv, dv, eps,
                  sigmoid=False):
    """Gated RMSNorm of x [rows, hv, dv] (storage array of x_dt, or float64 with
    x_dt = F64) with the gate z (token t's head h at z.flat[t*z_row_stride +
    h*dv + i]) and weight w [dv].  Returns y [rows, hv, dv] f64."""
    lib = _load()
    x = np.ascontiguousarray(x)
    z = np.ascontiguousarray(z)
    w = np.ascontiguousarray(w)
    y = np.zeros((rows, hv, dv), dtype=np.float64)
    rc = lib.oracle_rmsnorm_gated(rows, hv, dv, _p(x), x_dt, _p(z), z_dt, z_row_stride,
                                  _p(w), w_dt, float(eps), int(bool(sigmoid)), _p(y))
    if rc:
        raise OracleError(f"oracle_rmsnorm_gated: error {rc}")
    return y


# ---- convenience wrappers over the seeded workload cases ------------------
def decode_case(case, head_mask=None, rows=None, pool=None, state_dt=F32):
    """Oracle for a workloads.DecodeCase: gate then one recurrence step.
    `rows` (optional index array) restricts the batch to those rows; `pool`
    (stored as state_dt) replaces the case's f32 pool when given."""
    qv, kv, vv = case.q, case.k, case.v
    alpha, beta, idx = case.alpha, case.beta, case.idx
    qbuf, kbuf, vbuf = qv.buf, kv.buf, vv.buf
    if rows is not None:
        rows = np.asarray(rows)
        qbuf = np.ascontiguousarray(qbuf.reshape(case.batch, -1)[rows])
        kbuf = qbuf if kv.buf is qv.buf else np.ascontiguousarray(
            kbuf.reshape(case.batch, -1)[rows])
        vbuf = qbuf if vv.buf is qv.buf else np.ascontiguousarray(
            vbuf.reshape(case.batch, -1)[rows])
        alpha = np.ascontiguousarray(alpha[rows])
        beta = np.ascontiguousarray(beta[rows])
        idx = np.ascontiguousarray(idx[rows])
    batch = alpha.shape[0]
    g = gate(alpha, F32, case.dt_bias, case.ssm_a)
    return decode(batch=batch, hk=case.hk, hv=case.hv, dk=case.dk, dv=case.dv,
                  q=qbuf, q_off=qv.offset, q_rs=qv.row_stride,
                  k=kbuf, k_off=kv.offset, k_rs=kv.row_stride,
                  v=vbuf, v_off=vv.offset, v_rs=vv.row_stride, in_dt=case.in_dtype,
                  g=g, beta=beta, pool=case.pool if pool is None else pool, idx=idx,
                  scale=case.scale, l2_eps=case.l2_eps, l2norm=case.l2norm,
                  head_mask=head_mask, state_dt=state_dt)


def prefill_case(case, head_mask=None, pool=None, state_dt=F32):
    """Oracle for a workloads.PrefillCase: gate then the varlen recurrence;
    `pool` (stored as state_dt) replaces the case's f32 pool when given."""
    g = gate(case.alpha, F32, case.dt_bias, case.ssm_a)
    return prefill_varlen(cu_seqlens=case.cu_seqlens, hk=case.hk, hv=case.hv, dk=case.dk,
                          dv=case.dv, q=case.q.buf, q_off=case.q.offset, q_rs=case.q.row_stride,
                          k=case.k.buf, k_off=case.k.offset, k_rs=case.k.row_stride,
                          v=case.v.buf, v_off=case.v.offset, v_rs=case.v.row_stride,
                          in_dt=case.in_dtype, g=g, beta=case.beta,
                          pool=case.pool if pool is None else pool, idx=case.idx,
                          has_init=case.has_init, scale=case.scale, l2_eps=case.l2_eps,
                          l2norm=case.l2norm, head_mask=head_mask, state_dt=state_dt)


def _norm_rows(norm, total_rows, rows=None):
    z = norm.z
    assert z.offset == 0
    zbuf = z.buf.reshape(total_rows, z.row_stride)
    if rows is not None:
        zbuf = zbuf[np.asarray(rows)]
    return np.ascontiguousarray(zbuf)


def decode_norm_case(case, norm, *, sigmoid=False, rows=None, pool=None, state_dt=F32):
    """Oracle for a decode step followed by the gated RMSNorm of its f64
    outputs (workloads.NormInputs supplies z and w).  Returns (y, states)."""
    out, st = decode_case(case, rows=rows, pool=pool, state_dt=state_dt)
    zb = _norm_rows(norm, case.batch, rows)
    y = rmsnorm_gated(out, F64, zb, norm.dtype, norm.z.row_stride, norm.w, norm.dtype,
                      rows=out.shape[0], hv=case.hv, dv=case.dv, eps=norm.eps, sigmoid=sigmoid)
    return y, st


def prefill_norm_case(case, norm, *, sigmoid=False, head_mask=None):
    """Oracle for the varlen prefill followed by the gated RMSNorm of its f64
    outputs.  Returns (y, final states)."""
    out, st = prefill_case(case, head_mask=head_mask)
    zb = _norm_rows(norm, case.total_tokens)
    y = rmsnorm_gated(out, F64, zb, norm.dtype, norm.z.row_stride, norm.w, norm.dtype,
                      rows=out.shape[0], hv=case.hv, dv=case.dv, eps=norm.eps, sigmoid=sigmoid)
    return y, st


def conv1d_fwd(*, cu_seqlens, C, K, x, x_dt, x_rs, w, bias, state, st_dt, state_len,
               idx=None, has_init=None, silu=True):
    """Varlen depthwise causal conv.  x: storage buffer addressed as
    x.flat[t*x_rs + c]; w [C, K], bias [C] or None (x_dt); state [slots, C,
    state_len] (st_dt).  Returns (out [T, C] f64, new states [N, C, K-1] f64)."""
    lib = _load()
    cu = _need(np.asarray(cu_seqlens, dtype=np.int32), np.int32)
    n = cu.shape[0] - 1
    T = int(cu[-1])
    out = np.zeros((T, C), dtype=np.float64)
    st = np.zeros((n, C, max(K - 1, 0)), dtype=np.float64)
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    b = None if bias is None else np.ascontiguousarray(bias)
    state = np.ascontiguousarray(state)
    ia = None if idx is None else _need(np.asarray(idx, dtype=np.int32), np.int32)
    hi = None if has_init is None else _need(np.asarray(has_init, dtype=np.int8), np.int8)
    rc = lib.oracle_conv1d_fwd(n, _p(cu), C, K, _p(x), x_dt, x_rs, _p(w), _p(b), _p(state),
                               st_dt, state_len, state.shape[0], _p(ia), _p(hi), int(bool(silu)),
                               _p(out), _p(st))
    if rc:
        raise OracleError(f"oracle_conv1d_fwd: error {rc}")
    return out, st


def conv1d_update(*, batch, C, K, x, x_dt, x_rs, w, bias, state, st_dt, state_len, idx=None,
                  silu=True):
    """Single-token conv update.  Returns (out [B, C] f64, rolled states
    [B, C, K-1] f64, written [B] bool: False for rows with a negative slot)."""
    lib = _load()
    out = np.zeros((batch, C), dtype=np.float64)
    st = np.zeros((batch, C, max(K - 1, 0)), dtype=np.float64)
    wr = np.zeros(batch, dtype=np.int8)
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    b = None if bias is None else np.ascontiguousarray(bias)
    state = np.ascontiguousarray(state)
    ia = None if idx is None else _need(np.asarray(idx, dtype=np.int32), np.int32)
    rc = lib.oracle_conv1d_update(batch, C, K, _p(x), x_dt, x_rs, _p(w), _p(b), _p(state), st_dt,
                                  state_len, state.shape[0], _p(ia), int(bool(silu)), _p(out),
                                  _p(st), _p(wr))
    if rc:
        raise OracleError(f"oracle_conv1d_update: error {rc}")
    return out, st, wr.astype(bool)
