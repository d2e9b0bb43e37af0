"""MI355X-native fused attention (FlashAttention forward and backward on gfx950).

The compute lives in ``libfa.so`` (hand-written HIP kernels behind the C ABI
of ``include/fa.h``); this package only marshals torch tensors to it.
"""
from ._binding import (FAError, bwd, fwd, fwd_blocksparse, fwd_fp8, fwd_partial, fwd_splitkv, fwd_splitkv_noalloc,
                       load, merge, quant_fp8, quant_v_pow2, status_string)

__all__ = ["FAError", "bwd", "fwd", "fwd_blocksparse", "fwd_fp8", "fwd_partial", "fwd_splitkv", "fwd_splitkv_noalloc",
           "load", "merge", "quant_fp8", "quant_v_pow2", "status_string"]
