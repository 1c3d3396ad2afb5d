"""Gated DeltaNet hot path for AMD Instinct MI355X (gfx950).

The compute lives in libgdn.so (HIP kernels behind the C ABI of
include/gdn.h); ``gdn`` is its ctypes binding.  Importing this package loads
nothing; the first call loads the library and fails loudly if it is missing.
"""
from .gdn import (GDN_BF16, GDN_F16, GDN_F32, GdnError, conv1d_fwd, conv1d_update, decode,
                  decode_gated_norm, gate, gate_beta, load_library, post_conv, prefill_varlen,
                  prefill_varlen_gated, prefill_varlen_gated_norm, prefill_varlen_noalloc,
                  prefill_varlen_packed, prefill_workspace_size, rmsnorm_gated)

__all__ = ["GDN_BF16", "GDN_F16", "GDN_F32", "GdnError", "conv1d_fwd", "conv1d_update",
           "decode", "decode_gated_norm", "gate", "gate_beta", "load_library", "post_conv",
           "prefill_varlen", "prefill_varlen_gated", "prefill_varlen_gated_norm",
           "prefill_varlen_noalloc",
           "prefill_varlen_packed", "prefill_workspace_size", "rmsnorm_gated"]
