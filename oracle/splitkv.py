"""Attention over a key range and the merge of such partial results, in
float64 (test infrastructure only).

Ring attention (the "Flash Attention" tag page, excerpts on attention
variants and on ring attention) has every device compute attention of its
queries against one shard of the keys and values at a time and combine the
partial results; the combination itself is not spelled out on the pages.
The plain reading: a partial result over a key set J is the attention
restricted to J,

    O_J[i]   = sum_{j in J, visible} P_J[i, j] V[j],   P_J = softmax over J only
    lse_J[i] = ln sum_{j in J, visible} exp(S[i, j])   (-inf if no key is visible)

and, for disjoint key sets J_1..J_G covering all keys, the full result is

    lse[i] = ln sum_g exp(lse_g[i])
    O[i]   = sum_g exp(lse_g[i] - lse[i]) O_g[i]

because exp(lse_g) is exactly the part of the softmax denominator that J_g
contributes.  A part with lse_g = -inf contributes nothing; a row with every
part at -inf has O = 0 and lse = -inf.
"""
from __future__ import annotations

import numpy as np

from .attention import _as64, _row_chunks, scores_rows


def attention_partial(q, k, v, causal: bool, softmax_scale: float, kv_begin: int, kv_end: int):
    """O_J and lse_J for the key range J = [kv_begin, kv_end) (positions in the
    same sequence as the queries, so the causal mask uses them as they are)."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    if not 0 <= kv_begin <= kv_end <= N:
        raise ValueError("need 0 <= kv_begin <= kv_end <= N")
    O = np.zeros((B, H, N, d))
    lse = np.full((B, H, N), -np.inf)
    if kv_begin == kv_end:
        return O, lse
    rows = np.arange(N)
    keys = np.arange(kv_begin, kv_end)
    for b in range(B):
        for h in range(H):
            for rr in _row_chunks(rows, kv_end - kv_begin):
                S = scores_rows(q[b, h, rr], k[b, h, kv_begin:kv_end], softmax_scale)
                if causal:
                    S = np.where(keys[None, :] > rr[:, None], -np.inf, S)
                m = S.max(axis=1)
                live = np.isfinite(m)
                e = np.exp(S[live] - m[live, None])
                l = e.sum(axis=1)
                O[b, h, rr[live]] = (e / l[:, None]) @ v[b, h, kv_begin:kv_end]
                lse[b, h, rr[live]] = m[live] + np.log(l)
    return O, lse


def merge_partials(o_parts, lse_parts):
    """Combine partial results ``o_parts [G, ..., d]``, ``lse_parts [G, ...]``
    over disjoint key sets into (O, lse)."""
    o_parts, lse_parts = _as64(o_parts), _as64(lse_parts)
    m = lse_parts.max(axis=0)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe[None]), 0.0)
    s = w.sum(axis=0)
    lse = np.where(live, m_safe + np.log(np.where(live, s, 1.0)), -np.inf)
    coef = np.where(live[None], w / np.where(live, s, 1.0)[None], 0.0)
    O = (coef[..., None] * o_parts).sum(axis=0)
    return O, lse


def split_ranges(N: int, n_splits: int, align: int = 64):
    """Key ranges of a split into ``n_splits`` parts whose boundaries are
    multiples of ``align`` (the last part ends at N; trailing parts may be
    empty when N is short)."""
    tiles = -(-N // align)
    per = -(-tiles // n_splits)
    out = []
    for s in range(n_splits):
        lo = min(N, s * per * align)
        hi = min(N, (s + 1) * per * align)
        out.append((lo, hi))
    return out
