"""Block-sparse attention by its definition, in float64 (test infrastructure only).

The "Flash Attention" tag page (excerpt on attention variants) describes
block sparse attention: the attention matrix is cut into blocks and only
some blocks are computed -- full attention inside a block, sparse
connections between blocks.  The plain reading taken here: with a block
size of 64 queries by 64 keys and a 0/1 table ``mask[qb, kb]``,

    S[i, j] = softmax_scale * q_i . k_j   if mask[i // 64, j // 64] != 0
                                          (and j <= i when causal)
            = -inf                        otherwise

followed by the same row softmax, O = P V and lse as the dense definition
(``oracle.attention``).  A row whose blocks are all masked has no visible
key: it gets O = 0 and lse = -inf, the same convention as a partial result
over an empty key range.
"""
from __future__ import annotations

import numpy as np

from .attention import _as64, _row_chunks, scores_rows

BLOCK = 64


def expand_block_mask(mask: np.ndarray, N: int, block: int = BLOCK) -> np.ndarray:
    """Element mask [N, N] (True = visible) of a block table [ceil(N/block)]^2."""
    m = np.asarray(mask) != 0
    nb = -(-N // block)
    if m.shape != (nb, nb):
        raise ValueError(f"block mask must be {nb} x {nb} for N = {N}")
    idx = np.arange(N) // block
    return m[idx[:, None], idx[None, :]]


def attention_blocksparse(q, k, v, block_mask, causal: bool, softmax_scale: float, rows=None):
    """O and lse with a block mask.

    ``block_mask``: [nb, nb] shared by every (b, h), or [B, H, nb, nb].
    ``rows``: optional subset of query rows (every key is still considered).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    bm = np.asarray(block_mask)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((B, H, len(rows), d))
    lse = np.full((B, H, len(rows)), -np.inf)
    keys = np.arange(N)
    for b in range(B):
        for h in range(H):
            allow = expand_block_mask(bm if bm.ndim == 2 else bm[b, h], N)
            pos = 0
            for rr in _row_chunks(rows, N):
                S = scores_rows(q[b, h, rr], k[b, h], softmax_scale)
                vis = allow[rr]
                if causal:
                    vis = vis & (keys[None, :] <= rr[:, None])
                S = np.where(vis, S, -np.inf)
                m = S.max(axis=1)
                live = np.isfinite(m)
                e = np.exp(S[live] - m[live, None])
                l = e.sum(axis=1)
                idx = pos + np.nonzero(live)[0]
                O[b, h, idx] = (e / l[:, None]) @ v[b, h]
                lse[b, h, idx] = m[live] + np.log(l)
                pos += len(rr)
    return O, lse


def visible_pairs(block_mask, N: int, causal: bool, B: int = 1, H: int = 1) -> int:
    """Number of (query, key) pairs the block mask (and causal mask) leaves visible."""
    bm = np.asarray(block_mask)
    total = 0
    for b in range(B):
        for h in range(H):
            allow = expand_block_mask(bm if bm.ndim == 2 else bm[b, h], N)
            if causal:
                allow = np.tril(allow)
            total += int(allow.sum())
    return total
