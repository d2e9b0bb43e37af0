"""CPU oracle for the fused attention forward pass -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy code that states what the forward pass computes,
so the HIP path can be checked against it.  Only the test suite, the smoke
check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py``
may import it; the library and its Python binding never do, and this
package imports nothing from them.

Pages it follows (cited by title and section throughout):

* "From theory to implementation: the three FlashAttention generations
  dissected with Triton" (su666666.com news 140181) -- sections 2.1 (online
  softmax update), 3.1 (per-block causal mask), 4.1 (FP8 with dynamic
  scales).
* "Core principles behind FlashAttention's speed-up" (codearts.csdn.net)
  -- section 1.1 (tiled double loop), 1.2 (fused kernel), 1.3 (online softmax
  renormalisation), 4.2 (``softmax_scale = 1/sqrt(dim)``).
* "Flash Attention" tag page (guijiagi.com/tags/flash-attention) -- the
  excerpts on what FlashAttention solves (``S = QK^T/sqrt(d)``,
  ``P = softmax(S)``, ``O = PV``), on the performance bottleneck (online
  softmax over blocks, V2 deferred rescale) and on the standard attention
  listing (``(batch, heads, seq, dim)`` layout).

Modules:

* ``attention`` -- the definition: scores materialised in float64, explicit
  causal mask, two-pass softmax, ``O = P V`` and the per-row logsumexp.
* ``fp8`` -- the OCP e4m3fn codec, the per-64-row-tile dynamic scaling of Q
  and K, and the power-of-two per-(tile, column) scaling of V for FP8 P*V.
* ``online`` -- the pages' block-by-block online-softmax recurrences, used
  only to cross-check the two-pass definition.
* ``splitkv`` -- attention restricted to a key range (a partial result with
  its own lse) and the lse-weighted merge of partial results over disjoint
  key ranges (ring attention's combination step, split-KV on one device).
* ``blocksparse`` -- attention with a 64x64 block mask (only the blocks the
  table allows are computed), optionally combined with the causal mask.
* ``backward`` -- dQ, dK, dV of the forward definition for an upstream
  gradient dO (the chain rule through scores, softmax and the product with
  V), in full and for sampled query rows or key columns.
"""
from .attention import attention, attention_fp8, scores_rows
from .fp8 import (decode_e4m3, encode_e4m3, quantize_tiles, E4M3_MAX, TILE_ROWS, pow2_exponent,
                  quantize_v_pow2, dequantize_v_pow2)
from .online import online_softmax_attention, online_softmax_eager
from .backward import attention_backward, dq_rows, dkdv_cols
from .splitkv import attention_partial, merge_partials, split_ranges
from .blocksparse import attention_blocksparse, expand_block_mask, visible_pairs

__all__ = [
    "attention", "attention_fp8", "scores_rows",
    "decode_e4m3", "encode_e4m3", "quantize_tiles", "E4M3_MAX", "TILE_ROWS",
    "pow2_exponent", "quantize_v_pow2", "dequantize_v_pow2",
    "online_softmax_attention", "online_softmax_eager",
    "attention_backward", "dq_rows", "dkdv_cols",
    "attention_partial", "merge_partials", "split_ranges",
    "attention_blocksparse", "expand_block_mask", "visible_pairs",
]
