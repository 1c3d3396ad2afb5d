"""ctypes binding of libgdn (include/gdn.h): argument marshalling only.

Every step of the path runs in the HIP kernels of libgdn.so; this module turns
torch tensors into device pointers, element strides and dtype codes, passes
torch's current HIP stream, and raises ``GdnError`` on a non-zero return code.
There is no fallback: if the library is missing or fails to load, every entry
point raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_F16, GDN_BF16 = 0, 1, 2
GDN_L2NORM_QK = 1 << 0
GDN_CHECK_SLOTS = 1 << 1
GDN_PREFILL_SEQUENTIAL = 1 << 2
GDN_STATE_F16 = 1 << 3
GDN_STATE_BF16 = 1 << 4
GDN_NORM_SIGMOID = 1 << 5
GDN_BETA_ROUNDED = 1 << 7
GDN_CONV_SILU = 1 << 8
_STATE_FLAGS = {torch.float32: 0, torch.float16: GDN_STATE_F16, torch.bfloat16: GDN_STATE_BF16}

_TORCH_DT = {torch.float32: GDN_F32, torch.float16: GDN_F16, torch.bfloat16: GDN_BF16}

EXPORTS = ("gdn_conv1d_fwd", "gdn_conv1d_update", "gdn_gate", "gdn_gate_beta", "gdn_post_conv",
           "gdn_decode", "gdn_decode_packed", "gdn_decode_gated_norm",
           "gdn_rmsnorm_gated",
           "gdn_prefill_varlen_workspace_size", "gdn_prefill_varlen", "gdn_prefill_varlen_aux",
           "gdn_prefill_varlen_gated", "gdn_prefill_varlen_gated_norm", "gdn_prefill_varlen_packed",
           "gdn_prefill_varlen_noalloc",
           "gdn_last_error")


class GdnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libgdn.so and declare the C signatures (no GPU needed)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libgdn.so not built ({path}); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    vp, i64, f32, u32, i32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                  ctypes.c_uint32, ctypes.c_int, ctypes.c_size_t)
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_gate.restype = i32
    lib.gdn_gate.argtypes = [vp, i64, vp, i32, i64, vp, vp, i64, i64, vp]
    lib.gdn_decode.restype = i32
    lib.gdn_decode.argtypes = [vp, i32, vp, vp, vp, i32, i64, i64, i64, vp, i32, i64, vp, vp,
                               vp, i64, vp, i64, vp, i64, i64, i64, i64, i64, f32, f32, u32, vp]
    lib.gdn_decode_packed.restype = i32
    lib.gdn_decode_packed.argtypes = [vp, i32, vp, vp, vp, i32, i64, i64, i64, vp, vp, i32,
                                      i64, i64, vp, vp, vp, i64, vp, i64, i64, i64, i64, i64,
                                      f32, f32, u32, vp]
    lib.gdn_conv1d_fwd.restype = i32
    lib.gdn_conv1d_fwd.argtypes = [vp, i32, vp, i32, i64, vp, vp, vp, i64, i64, vp, vp, vp, i64,
                                   i64, i64, i64, u32, vp]
    lib.gdn_conv1d_update.restype = i32
    lib.gdn_conv1d_update.argtypes = [vp, i32, vp, i32, i64, vp, vp, vp, i64, i64, vp, i64, i64,
                                      i64, u32, vp]
    lib.gdn_gate_beta.restype = i32
    lib.gdn_gate_beta.argtypes = [vp, vp, i64, vp, vp, i32, i64, i64, vp, vp, i64, i64, u32, vp]
    lib.gdn_post_conv.restype = i32
    lib.gdn_post_conv.argtypes = [vp, vp, vp, i32, vp, vp, vp, i32, i64, vp, vp, i32, i64, i64,
                                  vp, vp, i64, i64, i64, i64, i64, f32, u32, vp]
    lib.gdn_decode_gated_norm.restype = i32
    lib.gdn_decode_gated_norm.argtypes = [vp, i32, vp, vp, vp, i32, i64, i64, i64, vp, i32, i64,
                                          vp, vp, vp, i64, vp, i64, vp, i64, i64, i64, i64, i64,
                                          f32, f32, vp, i64, vp, f32, u32, vp]
    lib.gdn_rmsnorm_gated.restype = i32
    lib.gdn_rmsnorm_gated.argtypes = [vp, i32, vp, i32, vp, i64, vp, i64, i64, i64, f32, u32,
                                      vp]
    lib.gdn_prefill_varlen_workspace_size.restype = sz
    lib.gdn_prefill_varlen_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, i32, u32]
    lib.gdn_prefill_varlen.restype = i32
    lib.gdn_prefill_varlen.argtypes = [vp, i32, vp, vp, vp, i32, i64, i64, i64, vp, i64, vp,
                                       i64, vp, i64, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                       f32, f32, u32, vp, sz, vp]
    lib.gdn_prefill_varlen_aux.restype = i32
    lib.gdn_prefill_varlen_aux.argtypes = lib.gdn_prefill_varlen.argtypes + [vp]
    pre = [vp, i32, vp, vp, vp, i32, i64, i64, i64]
    post = [vp, i64, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, f32, u32, vp, sz, vp, vp]
    lib.gdn_prefill_varlen_gated.restype = i32
    lib.gdn_prefill_varlen_gated.argtypes = pre + [vp, i32, i64, vp, vp, vp, i64] + post
    lib.gdn_prefill_varlen_gated_norm.restype = i32
    lib.gdn_prefill_varlen_gated_norm.argtypes = (pre + [vp, i32, i64, vp, vp, vp, i64] +
                                                  post[:13] + [vp, i64, vp, f32] + post[13:])
    lib.gdn_prefill_varlen_packed.restype = i32
    lib.gdn_prefill_varlen_packed.argtypes = pre + [vp, vp, i32, i64, i64, vp, vp] + post
    lib.gdn_prefill_varlen_noalloc.restype = i32
    lib.gdn_prefill_varlen_noalloc.argtypes = [vp, i32, vp, vp, vp, i32, i64, i64, i64, vp,
                                               i64, vp, i64, vp, i64, vp, vp, vp, i64, i64,
                                               i64, i64, i64, i64, f32, f32, u32, vp]
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise GdnError(rc, _lib.gdn_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    try:
        return _TORCH_DT[t.dtype]
    except KeyError:
        raise GdnError(-2, f"unsupported dtype {t.dtype}") from None


def _dev(t: Optional[torch.Tensor], name: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise GdnError(-1, f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise GdnError(-2, f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _rows(t: torch.Tensor, name: str, heads: int, dim: int) -> int:
    """Row stride (elements) of a [rows, heads, dim] (or [rows, heads*dim])
    operand whose rows are contiguous."""
    if t.dim() == 3:
        if t.shape[1] != heads or t.shape[2] != dim or t.stride(2) != 1 or t.stride(1) != dim:
            raise GdnError(-3, f"{name}: need [rows, {heads}, {dim}] with contiguous rows")
    elif t.dim() == 2:
        if t.shape[1] != heads * dim or t.stride(1) != 1:
            raise GdnError(-3, f"{name}: need [rows, {heads * dim}] with contiguous rows")
    else:
        raise GdnError(-3, f"{name}: rank {t.dim()} not supported")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), heads * dim)


def _rows2(t: torch.Tensor, name: str, width: int) -> int:
    if t.dim() != 2 or t.shape[1] != width or t.stride(1) != 1:
        raise GdnError(-3, f"{name}: need [rows, {width}] with contiguous rows")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), width)


def _state_flags(pool: torch.Tensor) -> int:
    try:
        return _STATE_FLAGS[pool.dtype]
    except KeyError:
        raise GdnError(-2, f"state_pool dtype {pool.dtype} not supported") from None


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _new(shape, dtype, device, stream) -> torch.Tensor:
    """A tensor the binding allocates for a call.  When the call runs on a
    stream other than the current one, the caching allocator is told that the
    memory is in use on that stream, so it is not handed to other work before
    the call's kernels are done with it."""
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        t.record_stream(stream)
    return t


def gate(alpha: torch.Tensor, dt_bias: torch.Tensor, ssm_a: torch.Tensor,
         out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """g[r, h] = softplus(alpha[r, h] + dt_bias[h]) * ssm_a[h]  ->  [rows, hv] f32."""
    lib = load_library()
    rows, hv = alpha.shape[0], dt_bias.shape[0]
    a_rs = _rows2(alpha, "alpha", hv)
    if out is None:
        out = _new((rows, hv), torch.float32, alpha.device, stream)
    g_rs = _rows2(out, "g", hv)
    _check(lib.gdn_gate(_dev(out, "g", torch.float32), g_rs, _dev(alpha, "alpha"), _dt(alpha),
                        a_rs, _dev(dt_bias, "dt_bias", torch.float32),
                        _dev(ssm_a, "ssm_a", torch.float32), rows, hv, _stream(stream)))
    return out


def decode(q, k, v, alpha, dt_bias, ssm_a, beta, state_pool, state_idx, *, scale: float,
           l2norm: bool = True, l2_eps: float = 1e-6, out: Optional[torch.Tensor] = None,
           out_dtype=None, check_slots: bool = False, beta_raw: bool = False,
           stream=None) -> torch.Tensor:
    """One decode step, gate fused, pool updated in place.

    q, k: [B, Hk, Dk]; v: [B, Hv, Dv] (rows may be strided, e.g. views into one
    packed q|k|v buffer); alpha [B, Hv]; dt_bias, ssm_a [Hv] f32; beta [B, Hv] f32;
    state_pool [slots, Hv, Dv, Dk] contiguous, f32 or 16-bit storage (float16 /
    bfloat16: widened to f32 for the step, the new state rounded on store);
    state_idx [B] int32.  check_slots: validate state_idx first (GDN_CHECK_SLOTS:
    reads it back and waits on the stream; not capturable).  beta_raw: alpha
    and beta are the raw projections a and b in one dtype (gdn_decode_packed:
    beta = sigmoid(b) rounded through that dtype)."""
    return _decode(q, k, v, alpha, dt_bias, ssm_a, beta, state_pool, state_idx, scale=scale,
                   l2norm=l2norm, l2_eps=l2_eps, out=out, out_dtype=out_dtype,
                   check_slots=check_slots, beta_raw=beta_raw, stream=stream, norm=None)


def decode_gated_norm(q, k, v, alpha, dt_bias, ssm_a, beta, state_pool, state_idx, norm_z,
                      norm_w, *, scale: float, norm_eps: float = 1e-6, sigmoid: bool = False,
                      l2norm: bool = True, l2_eps: float = 1e-6,
                      out: Optional[torch.Tensor] = None, out_dtype=None,
                      check_slots: bool = False, beta_raw: bool = False,
                      stream=None) -> torch.Tensor:
    """decode() with the gated RMSNorm fused after the step:
    out = o / sqrt(mean(o^2) + norm_eps) * norm_w * act(norm_z), act = silu or
    sigmoid.  norm_z: [B, Hv, Dv] (rows may be padded views of a wider
    buffer) and norm_w: [Dv], both in q's dtype."""
    return _decode(q, k, v, alpha, dt_bias, ssm_a, beta, state_pool, state_idx, scale=scale,
                   l2norm=l2norm, l2_eps=l2_eps, out=out, out_dtype=out_dtype,
                   check_slots=check_slots, beta_raw=beta_raw, stream=stream,
                   norm=(norm_z, norm_w, norm_eps, sigmoid))


def _decode(q, k, v, alpha, dt_bias, ssm_a, beta, state_pool, state_idx, *, scale, l2norm,
            l2_eps, out, out_dtype, check_slots, beta_raw, stream, norm):
    lib = load_library()
    if state_pool.dim() != 4 or not state_pool.is_contiguous():
        raise GdnError(-3, "state_pool: need contiguous [slots, Hv, Dv, Dk]")
    slots, hv, dv, dk = state_pool.shape
    B = state_idx.shape[0]
    hk = q.shape[1] if q.dim() == 3 else q.shape[1] // dk
    q_rs = _rows(q, "q", hk, dk)
    k_rs = _rows(k, "k", hk, dk)
    v_rs = _rows(v, "v", hv, dv)
    a_rs = _rows2(alpha, "alpha", hv)
    b_rs = _rows2(beta, "beta", hv)
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta)):
        if t.shape[0] != B:
            raise GdnError(-3, f"{name}: {t.shape[0]} rows, state_idx has {B}")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise GdnError(-2, "q, k, v must share a dtype")
    if out is None:
        out = _new((B, hv, dv), out_dtype or q.dtype, q.device, stream)
    if not out.is_contiguous() or tuple(out.shape) != (B, hv, dv):
        raise GdnError(-3, "out: need contiguous [B, Hv, Dv]")
    flags = ((GDN_L2NORM_QK if l2norm else 0) | (GDN_CHECK_SLOTS if check_slots else 0) |
             _state_flags(state_pool))
    head = [_dev(out, "out"), _dt(out), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dt(q),
            q_rs, k_rs, v_rs]
    tail = [_dev(state_pool, "state_pool"), slots, _dev(state_idx, "state_idx", torch.int32),
            B, hk, hv, dk, dv, float(scale), float(l2_eps)]
    if beta_raw:
        if norm is not None:
            raise GdnError(-1, "the fused norm takes post-sigmoid beta")
        _check(lib.gdn_decode_packed(*head, _dev(alpha, "a"), _dev(beta, "b", alpha.dtype),
                                     _dt(alpha), a_rs, b_rs,
                                     _dev(dt_bias, "dt_bias", torch.float32),
                                     _dev(ssm_a, "ssm_a", torch.float32), *tail, flags,
                                     _stream(stream)))
        return out
    args = head + [_dev(alpha, "alpha"), _dt(alpha), a_rs,
                   _dev(dt_bias, "dt_bias", torch.float32), _dev(ssm_a, "ssm_a", torch.float32),
                   _dev(beta, "beta", torch.float32), b_rs] + tail
    if norm is None:
        _check(lib.gdn_decode(*args, flags, _stream(stream)))
        return out
    z, w, eps, sigmoid = norm
    if z.shape[0] != B:
        raise GdnError(-3, f"norm_z: {z.shape[0]} rows, state_idx has {B}")
    z_rs = _rows(z, "norm_z", hv, dv)
    if w.dim() != 1 or w.shape[0] != dv or not w.is_contiguous():
        raise GdnError(-3, f"norm_w: need contiguous [{dv}]")
    flags |= GDN_NORM_SIGMOID if sigmoid else 0
    _check(lib.gdn_decode_gated_norm(*args, _dev(z, "norm_z", q.dtype), z_rs,
                                     _dev(w, "norm_w", q.dtype), float(eps), flags,
                                     _stream(stream)))
    return out


def _conv_common(x, weight, conv_state, name):
    if x.dim() != 2 or x.stride(1) != 1:
        raise GdnError(-3, f"{name}: x needs [rows, C] with contiguous rows")
    rows, C = x.shape
    x_rs = x.stride(0) if rows > 1 else max(x.stride(0), C)
    if weight.dim() != 2 or weight.shape[0] != C or not weight.is_contiguous():
        raise GdnError(-3, f"{name}: weight needs contiguous [C, K]")
    K = weight.shape[1]
    if conv_state is None:
        return rows, C, x_rs, K, 0, 0, 0
    if conv_state.dim() != 3 or conv_state.shape[1] != C or not conv_state.is_contiguous():
        raise GdnError(-3, f"{name}: conv_state needs contiguous [slots, C, state_len]")
    return rows, C, x_rs, K, conv_state.shape[2], conv_state.shape[0], _state_flags(conv_state)


def conv1d_fwd(x, weight, bias, conv_state, cu_seqlens, *, state_idx=None,
               has_initial_state=None, silu: bool = True, out=None, out_dtype=None,
               check_slots: bool = False, stream=None) -> torch.Tensor:
    """Depthwise causal conv over sequences packed back to back: x [T, C]
    (rows may be strided), weight [C, K], bias [C] or None, conv_state
    [slots, C, state_len] (f32/f16/bf16, read then written back in place)."""
    lib = load_library()
    T, C, x_rs, K, sl, slots, sflags = _conv_common(x, weight, conv_state, "conv1d_fwd")
    N = cu_seqlens.shape[0] - 1
    if out is None:
        out = _new((T, C), out_dtype or x.dtype, x.device, stream)
    if not out.is_contiguous() or tuple(out.shape) != (T, C):
        raise GdnError(-3, "out: need contiguous [T, C]")
    flags = (GDN_CONV_SILU if silu else 0) | (GDN_CHECK_SLOTS if check_slots else 0) | sflags
    _check(lib.gdn_conv1d_fwd(_dev(out, "out"), _dt(out), _dev(x, "x"), _dt(x), x_rs,
                              _dev(weight, "weight", x.dtype), _dev(bias, "bias", x.dtype),
                              _dev(conv_state, "conv_state"), sl, slots,
                              _dev(state_idx, "state_idx", torch.int32),
                              _dev(has_initial_state, "has_initial_state", torch.int8),
                              _dev(cu_seqlens, "cu_seqlens", torch.int32), N, T, C, K, flags,
                              _stream(stream)))
    return out


def conv1d_update(x, weight, bias, conv_state, *, state_idx=None, silu: bool = True, out=None,
                  out_dtype=None, check_slots: bool = False, stream=None) -> torch.Tensor:
    """One token per row through the conv: x [B, C] (rows may be strided), the
    state rows (state_idx [B] int32 or None: row r) rolled in place."""
    lib = load_library()
    B, C, x_rs, K, sl, slots, sflags = _conv_common(x, weight, conv_state, "conv1d_update")
    if out is None:
        out = _new((B, C), out_dtype or x.dtype, x.device, stream)
    if not out.is_contiguous() or tuple(out.shape) != (B, C):
        raise GdnError(-3, "out: need contiguous [B, C]")
    flags = (GDN_CONV_SILU if silu else 0) | (GDN_CHECK_SLOTS if check_slots else 0) | sflags
    _check(lib.gdn_conv1d_update(_dev(out, "out"), _dt(out), _dev(x, "x"), _dt(x), x_rs,
                                 _dev(weight, "weight", x.dtype), _dev(bias, "bias", x.dtype),
                                 _dev(conv_state, "conv_state"), sl, slots,
                                 _dev(state_idx, "state_idx", torch.int32), B, C, K, flags,
                                 _stream(stream)))
    return out


def gate_beta(a, b, dt_bias, ssm_a, *, rounded: bool = False, g=None, beta=None,
              stream=None):
    """g = softplus(a + dt_bias) * ssm_a and beta = sigmoid(b) ([rows, hv] f32 each)
    from raw a and b ([rows, hv], one dtype, rows may be strided: e.g. column
    views of one merged b|a row).  rounded: beta rounded through b's dtype."""
    lib = load_library()
    rows, hv = a.shape[0], dt_bias.shape[0]
    a_rs = _rows2(a, "a", hv)
    b_rs = _rows2(b, "b", hv)
    if b.shape[0] != rows:
        raise GdnError(-3, f"b: {b.shape[0]} rows, a has {rows}")
    if g is None:
        g = _new((rows, hv), torch.float32, a.device, stream)
    if beta is None:
        beta = _new((rows, hv), torch.float32, a.device, stream)
    for name, t in (("g", g), ("beta", beta)):
        if not t.is_contiguous() or tuple(t.shape) != (rows, hv):
            raise GdnError(-3, f"{name}: need contiguous [{rows}, {hv}]")
    _check(lib.gdn_gate_beta(_dev(g, "g", torch.float32), _dev(beta, "beta", torch.float32), hv,
                             _dev(a, "a"), _dev(b, "b", a.dtype), _dt(a), a_rs, b_rs,
                             _dev(dt_bias, "dt_bias", torch.float32),
                             _dev(ssm_a, "ssm_a", torch.float32), rows, hv,
                             GDN_BETA_ROUNDED if rounded else 0, _stream(stream)))
    return g, beta


def post_conv(conv, a, b, dt_bias, ssm_a, *, hk: int, dk: int, dv: int, l2_eps: float = 1e-6,
              out_dtype=None, rounded: bool = False, stream=None):
    """The post-conv front-end: conv [T, >= 2*hk*dk + hv*dv] (rows contiguous, may
    be padded) -> (q, k [T, hk, dk] normalised, v [T, hv, dv], g, beta [T, hv])."""
    lib = load_library()
    T = conv.shape[0]
    hv = dt_bias.shape[0]
    if conv.dim() != 2 or conv.stride(1) != 1 or conv.shape[1] < 2 * hk * dk + hv * dv:
        raise GdnError(-3, "conv: need [T, >= 2*hk*dk + hv*dv] with contiguous rows")
    conv_rs = conv.stride(0) if T > 1 else max(conv.stride(0), conv.shape[1])
    a_rs = _rows2(a, "a", hv)
    b_rs = _rows2(b, "b", hv)
    od = out_dtype or conv.dtype
    q = _new((T, hk, dk), od, conv.device, stream)
    k = _new((T, hk, dk), od, conv.device, stream)
    v = _new((T, hv, dv), od, conv.device, stream)
    g = _new((T, hv), torch.float32, conv.device, stream)
    beta = _new((T, hv), torch.float32, conv.device, stream)
    _check(lib.gdn_post_conv(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dt(q), _dev(g, "g"),
                             _dev(beta, "beta"), _dev(conv, "conv"), _dt(conv), conv_rs,
                             _dev(a, "a"), _dev(b, "b", a.dtype), _dt(a), a_rs, b_rs,
                             _dev(dt_bias, "dt_bias", torch.float32),
                             _dev(ssm_a, "ssm_a", torch.float32), T, hk, hv, dk, dv,
                             float(l2_eps), GDN_BETA_ROUNDED if rounded else 0,
                             _stream(stream)))
    return q, k, v, g, beta


def rmsnorm_gated(x, z, w, *, eps: float = 1e-6, sigmoid: bool = False,
                  out: Optional[torch.Tensor] = None, out_dtype=None,
                  stream=None) -> torch.Tensor:
    """Gated RMSNorm: out = x / sqrt(mean(x^2) + eps) * w * act(z) per
    (row, head), act = silu or sigmoid.  x: [T, Hv, Dv] contiguous; z: [T, Hv, Dv]
    (rows may be padded views of a wider buffer); w: [Dv]; all one dtype."""
    lib = load_library()
    if x.dim() != 3 or not x.is_contiguous():
        raise GdnError(-3, "x: need contiguous [T, Hv, Dv]")
    T, hv, dv = x.shape
    if z.shape[0] != T:
        raise GdnError(-3, f"z: {z.shape[0]} rows, x has {T}")
    z_rs = _rows(z, "z", hv, dv)
    if w.dim() != 1 or w.shape[0] != dv or not w.is_contiguous():
        raise GdnError(-3, f"w: need contiguous [{dv}]")
    if out is None:
        out = _new((T, hv, dv), out_dtype or x.dtype, x.device, stream)
    if not out.is_contiguous() or tuple(out.shape) != (T, hv, dv):
        raise GdnError(-3, "out: need contiguous [T, Hv, Dv]")
    _check(lib.gdn_rmsnorm_gated(_dev(out, "out"), _dt(out), _dev(x, "x"), _dt(x),
                                 _dev(z, "z", x.dtype), z_rs, _dev(w, "w", x.dtype), T, hv, dv,
                                 float(eps), GDN_NORM_SIGMOID if sigmoid else 0,
                                 _stream(stream)))
    return out


def prefill_workspace_size(total_tokens, num_seqs, hk, hv, dk, dv, in_dtype,
                           sequential=False, l2norm=True) -> int:
    lib = load_library()
    flags = (GDN_L2NORM_QK if l2norm else 0) | (GDN_PREFILL_SEQUENTIAL if sequential else 0)
    return lib.gdn_prefill_varlen_workspace_size(total_tokens, num_seqs, hk, hv, dk, dv,
                                                 _TORCH_DT[in_dtype], flags)


def _prefill_common(q, k, v, state_pool, cu_seqlens, scale, state_idx, has_initial_state,
                    l2norm, l2_eps, out, out_dtype, sequential, check_slots, stream,
                    extra_flags=0):
    """The arguments before and after the gate inputs of every prefill entry."""
    if state_pool.dim() != 4 or not state_pool.is_contiguous():
        raise GdnError(-3, "state_pool: need contiguous [slots, Hv, Dv, Dk]")
    slots, hv, dv, dk = state_pool.shape
    T = q.shape[0]
    N = cu_seqlens.shape[0] - 1
    hk = q.shape[1] if q.dim() == 3 else q.shape[1] // dk
    q_rs = _rows(q, "q", hk, dk)
    k_rs = _rows(k, "k", hk, dk)
    v_rs = _rows(v, "v", hv, dv)
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise GdnError(-2, "q, k, v must share a dtype")
    if out is None:
        out = _new((T, hv, dv), out_dtype or q.dtype, q.device, stream)
    if not out.is_contiguous() or tuple(out.shape) != (T, hv, dv):
        raise GdnError(-3, "out: need contiguous [T, Hv, Dv]")
    flags = ((GDN_L2NORM_QK if l2norm else 0) | (GDN_PREFILL_SEQUENTIAL if sequential else 0) |
             (GDN_CHECK_SLOTS if check_slots else 0) | _state_flags(state_pool) | extra_flags)
    head = [_dev(out, "out"), _dt(out), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dt(q),
            q_rs, k_rs, v_rs]
    tail = [_dev(state_pool, "state_pool"), slots,
            _dev(state_idx, "state_idx", torch.int32),
            _dev(has_initial_state, "has_initial_state", torch.int8),
            _dev(cu_seqlens, "cu_seqlens", torch.int32), N, T, hk, hv, dk, dv, float(scale),
            float(l2_eps), flags]
    return out, head, tail, (T, N, hk, hv, dk, dv, _dt(q), flags)


def _workspace(lib, ws_key, workspace, device, stream):
    """The call's workspace (the caller's when large enough, else a new one),
    its address and size.  The caller keeps the returned tensor referenced
    until the launch has been enqueued: freed earlier, the caching allocator
    would mark it free on `stream` before the kernels that use it, and could
    hand it to other work while they run."""
    ws_need = lib.gdn_prefill_varlen_workspace_size(*ws_key)
    if ws_need and (workspace is None or workspace.numel() * workspace.element_size() < ws_need):
        workspace = _new((ws_need,), torch.uint8, device, stream)
    ws_ptr = _dev(workspace, "workspace") if ws_need else None
    ws_bytes = workspace.numel() * workspace.element_size() if ws_need else 0
    return workspace, ws_ptr, ws_bytes


def prefill_varlen(q, k, v, g, beta, state_pool, cu_seqlens, *, scale: float,
                   state_idx: Optional[torch.Tensor] = None,
                   has_initial_state: Optional[torch.Tensor] = None, l2norm: bool = True,
                   l2_eps: float = 1e-6, out: Optional[torch.Tensor] = None, out_dtype=None,
                   sequential: bool = False, workspace: Optional[torch.Tensor] = None,
                   check_slots: bool = False, stream=None, aux_stream=None) -> torch.Tensor:
    """Varlen prefill over sequences packed back to back (cu_seqlens [N+1] int32).

    q, k: [T, Hk, Dk]; v: [T, Hv, Dv]; g, beta: [T, Hv] f32; state_pool
    [slots, Hv, Dv, Dk] f32, float16 or bfloat16 (initial states read, final
    states written).  check_slots: validate cu_seqlens and state_idx first
    (GDN_CHECK_SLOTS: reads them back and waits on the stream).  aux_stream:
    a second stream of the caller's for the split schedule
    (gdn_prefill_varlen_aux); without it the call runs on `stream` alone."""
    lib = load_library()
    out, head, tail, ws_key = _prefill_common(q, k, v, state_pool, cu_seqlens, scale, state_idx,
                                              has_initial_state, l2norm, l2_eps, out, out_dtype,
                                              sequential, check_slots, stream)
    hv = state_pool.shape[1]
    gate = [_dev(g, "g", torch.float32), _rows2(g, "g", hv), _dev(beta, "beta", torch.float32),
            _rows2(beta, "beta", hv)]
    workspace, ws_ptr, ws_bytes = _workspace(lib, ws_key, workspace, q.device, stream)
    if aux_stream is not None:
        _check(lib.gdn_prefill_varlen_aux(*head, *gate, *tail, ws_ptr, ws_bytes, _stream(stream),
                                          aux_stream.cuda_stream))
    else:
        _check(lib.gdn_prefill_varlen(*head, *gate, *tail, ws_ptr, ws_bytes, _stream(stream)))
    return out


def prefill_varlen_gated(q, k, v, alpha, dt_bias, ssm_a, beta, state_pool, cu_seqlens, *,
                         scale: float, state_idx=None, has_initial_state=None,
                         l2norm: bool = True, l2_eps: float = 1e-6, out=None, out_dtype=None,
                         sequential: bool = False, workspace=None, check_slots: bool = False,
                         stream=None, aux_stream=None) -> torch.Tensor:
    """prefill_varlen with the gate fused (gdn_prefill_varlen_gated): alpha
    [T, Hv] (f32/f16/bf16, rows may be strided), dt_bias and ssm_a [Hv] f32,
    beta [T, Hv] f32 post-sigmoid; no g array is formed."""
    lib = load_library()
    out, head, tail, ws_key = _prefill_common(q, k, v, state_pool, cu_seqlens, scale, state_idx,
                                              has_initial_state, l2norm, l2_eps, out, out_dtype,
                                              sequential, check_slots, stream)
    hv = state_pool.shape[1]
    gate = [_dev(alpha, "alpha"), _dt(alpha), _rows2(alpha, "alpha", hv),
            _dev(dt_bias, "dt_bias", torch.float32), _dev(ssm_a, "ssm_a", torch.float32),
            _dev(beta, "beta", torch.float32), _rows2(beta, "beta", hv)]
    workspace, ws_ptr, ws_bytes = _workspace(lib, ws_key, workspace, q.device, stream)
    _check(lib.gdn_prefill_varlen_gated(*head, *gate, *tail, ws_ptr, ws_bytes, _stream(stream),
                                        aux_stream.cuda_stream if aux_stream is not None
                                        else None))
    return out


def prefill_varlen_gated_norm(q, k, v, alpha, dt_bias, ssm_a, beta, state_pool, cu_seqlens,
                              norm_z, norm_w, *, scale: float, norm_eps: float = 1e-6,
                              sigmoid: bool = False, state_idx=None, has_initial_state=None,
                              l2norm: bool = True, l2_eps: float = 1e-6, out=None,
                              sequential: bool = False, workspace=None,
                              check_slots: bool = False, stream=None,
                              aux_stream=None) -> torch.Tensor:
    """prefill_varlen_gated, then the gated RMSNorm over the output in place
    (gdn_prefill_varlen_gated_norm): out = o / sqrt(mean(o^2) + norm_eps) *
    norm_w * act(norm_z), act = silu or sigmoid.  norm_z: [T, Hv, Dv] (rows
    may be padded views of a wider buffer) and norm_w: [Dv], both in q's
    dtype, which is also the output's."""
    lib = load_library()
    out, head, tail, ws_key = _prefill_common(q, k, v, state_pool, cu_seqlens, scale, state_idx,
                                              has_initial_state, l2norm, l2_eps, out, None,
                                              sequential, check_slots, stream)
    hv, dv = state_pool.shape[1], state_pool.shape[2]
    gate = [_dev(alpha, "alpha"), _dt(alpha), _rows2(alpha, "alpha", hv),
            _dev(dt_bias, "dt_bias", torch.float32), _dev(ssm_a, "ssm_a", torch.float32),
            _dev(beta, "beta", torch.float32), _rows2(beta, "beta", hv)]
    if norm_z.dtype != q.dtype or norm_w.dtype != q.dtype:
        raise GdnError(-2, "norm_z and norm_w must have q's dtype")
    if norm_w.dim() != 1 or norm_w.shape[0] != dv or not norm_w.is_contiguous():
        raise GdnError(-3, "norm_w: need contiguous [Dv]")
    norm = [_dev(norm_z, "norm_z"), _rows(norm_z, "norm_z", hv, dv), _dev(norm_w, "norm_w"),
            float(norm_eps)]
    flags = tail[-1] | (GDN_NORM_SIGMOID if sigmoid else 0)
    workspace, ws_ptr, ws_bytes = _workspace(lib, ws_key, workspace, q.device, stream)
    _check(lib.gdn_prefill_varlen_gated_norm(*head, *gate, *tail[:-1], *norm, flags, ws_ptr,
                                             ws_bytes, _stream(stream),
                                             aux_stream.cuda_stream if aux_stream is not None
                                             else None))
    return out


def prefill_varlen_packed(q, k, v, a, b, dt_bias, ssm_a, state_pool, cu_seqlens, *,
                          scale: float, rounded: bool = False, state_idx=None,
                          has_initial_state=None, l2norm: bool = True, l2_eps: float = 1e-6,
                          out=None, out_dtype=None, sequential: bool = False, workspace=None,
                          check_slots: bool = False, stream=None,
                          aux_stream=None) -> torch.Tensor:
    """The prefill fed by the front-end's raw projections
    (gdn_prefill_varlen_packed): q, k, v may be views into the conv output rows;
    a, b [T, Hv] raw (one dtype, rows may be strided: column views of one
    merged b|a row); g and beta = sigmoid(b) (rounded through b's dtype with
    `rounded`) are formed in the kernels."""
    lib = load_library()
    out, head, tail, ws_key = _prefill_common(
        q, k, v, state_pool, cu_seqlens, scale, state_idx, has_initial_state, l2norm, l2_eps, out,
        out_dtype, sequential, check_slots, stream, GDN_BETA_ROUNDED if rounded else 0)
    hv = state_pool.shape[1]
    if b.shape[0] != a.shape[0]:
        raise GdnError(-3, f"b: {b.shape[0]} rows, a has {a.shape[0]}")
    gate = [_dev(a, "a"), _dev(b, "b", a.dtype), _dt(a), _rows2(a, "a", hv), _rows2(b, "b", hv),
            _dev(dt_bias, "dt_bias", torch.float32), _dev(ssm_a, "ssm_a", torch.float32)]
    workspace, ws_ptr, ws_bytes = _workspace(lib, ws_key, workspace, q.device, stream)
    _check(lib.gdn_prefill_varlen_packed(*head, *gate, *tail, ws_ptr, ws_bytes, _stream(stream),
                                         aux_stream.cuda_stream if aux_stream is not None
                                         else None))
    return out


NOALLOC_SCRATCH_BYTES = 128 << 20   # GDN_NOALLOC_SCRATCH_BYTES of include/gdn.h


def prefill_varlen_noalloc(q, k, v, g, beta, state_pool, cu_seqlens, *, scale: float,
                           state_idx: Optional[torch.Tensor] = None,
                           has_initial_state: Optional[torch.Tensor] = None,
                           l2norm: bool = True, l2_eps: float = 1e-6,
                           out: Optional[torch.Tensor] = None, out_dtype=None,
                           sequential: bool = False, check_slots: bool = False,
                           stream=None) -> torch.Tensor:
    """prefill_varlen through gdn_prefill_varlen_noalloc: no workspace; the
    library's fixed per-device scratch holds the per-call records (calls that
    overlap on one device race on it).  Pass `out` to allocate nothing here."""
    lib = load_library()
    out, head, tail, _ = _prefill_common(q, k, v, state_pool, cu_seqlens, scale, state_idx,
                                         has_initial_state, l2norm, l2_eps, out, out_dtype,
                                         sequential, check_slots, stream)
    hv = state_pool.shape[1]
    gate = [_dev(g, "g", torch.float32), _rows2(g, "g", hv), _dev(beta, "beta", torch.float32),
            _rows2(beta, "beta", hv)]
    _check(lib.gdn_prefill_varlen_noalloc(*head, *gate, *tail, _stream(stream)))
    return out
