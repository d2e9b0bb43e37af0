"""Attention forward by its definition, in float64 (test infrastructure only).

For every (batch b, head h) and query row i:

    S[i, j]  = softmax_scale * sum_k Q[i, k] K[j, k]
    S[i, j]  = -inf  where causal and j > i
    m_i      = max_j S[i, j]
    e[i, j]  = exp(S[i, j] - m_i),   l_i = sum_j e[i, j]
    P[i, j]  = e[i, j] / l_i
    O[i, :]  = sum_j P[i, j] V[j, :]
    lse_i    = m_i + ln(l_i)

Sources: the "Flash Attention" tag page (excerpt on what FlashAttention
solves: scores, softmax, product with V; excerpt with the standard
attention listing: ``(batch, heads, seq, dim)``); "Core principles behind
FlashAttention's speed-up" section 4.2 (``softmax_scale``, default
``1/sqrt(dim)``); the Triton walkthrough page section 3.1 (causal mask keeps
key positions at or before the query position; the comparison operator is
lost in the page text, and the reading "key j <= query i" is taken).
The logsumexp is not named on the pages; it is the per-row statistic that
the recomputing backward pass of the walkthrough's section 2.2 needs.

The whole score row is materialised (rows are processed in chunks only to
bound memory; every chunk holds complete rows, so the softmax is the plain
two-pass one).  numpy's matmul is the only library primitive used.
"""
from __future__ import annotations

import numpy as np

_CHUNK_ELEMS = 1 << 22   # scores per chunk (32 MiB of float64)


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _softmax_rows(S: np.ndarray, V: np.ndarray):
    """Two-pass softmax over whole rows of S, then P @ V.  Returns (O, lse)."""
    m = S.max(axis=1)
    e = np.exp(S - m[:, None])
    l = e.sum(axis=1)
    P = e / l[:, None]
    O = P @ V
    lse = m + np.log(l)
    return O, lse


def _causal_mask(S: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Set S[r, j] = -inf where key j comes after query rows[r]."""
    cols = np.arange(S.shape[1])
    return np.where(cols[None, :] > rows[:, None], -np.inf, S)


def scores_rows(q_rows, k, softmax_scale):
    """Scaled scores of the given query rows against every key: [R, N]."""
    return softmax_scale * (_as64(q_rows) @ _as64(k).T)


def _row_chunks(rows: np.ndarray, n_keys: int):
    step = max(1, _CHUNK_ELEMS // max(1, n_keys))
    for s in range(0, len(rows), step):
        yield rows[s:s + step]


def attention(q, k, v, causal: bool, softmax_scale: float, rows=None):
    """O and lse of softmax(softmax_scale * Q K^T [causally masked]) V.

    q, k, v: arrays ``[B, H, N, d]`` holding exactly the values the device
    receives (they are widened to float64 here).  ``rows``: optional 1-D
    array of query indices; only those rows are computed (every key is
    still used).  Returns ``O [B, H, R, d]`` and ``lse [B, H, R]`` in
    float64 with R = N or ``len(rows)``.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    if k.shape != (B, H, N, d) or v.shape != (B, H, N, d):
        raise ValueError("q, k, v must share the shape [B, H, N, d]")
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.empty((B, H, len(rows), d))
    lse = np.empty((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            pos = 0
            for rr in _row_chunks(rows, N):
                S = scores_rows(q[b, h, rr], k[b, h], softmax_scale)
                if causal:
                    S = _causal_mask(S, rr)
                o, s = _softmax_rows(S, v[b, h])
                O[b, h, pos:pos + len(rr)] = o
                lse[b, h, pos:pos + len(rr)] = s
                pos += len(rr)
    return O, lse


def attention_fp8(q_vals, q_scale, k_vals, k_scale, v, causal: bool,
                  softmax_scale: float, tile_rows: int = 64, rows=None):
    """Attention on FP8-quantised Q and K with per-tile scales.

    ``q_vals``/``k_vals`` are the decoded e4m3 values ``[B, H, N, d]``
    (see ``oracle.fp8``), ``q_scale``/``k_scale`` the float32 scale of
    every ``tile_rows``-row tile ``[B, H, ceil(N/tile_rows)]``.  As in the
    Triton walkthrough's section 4.1, the dot product of the quantised
    operands is taken in full precision and multiplied by
    ``1 / (q_scale * k_scale)`` to undo the scaling; everything after that
    is the plain definition above.  All in float64.
    """
    qv, kv, v = _as64(q_vals), _as64(k_vals), _as64(v)
    qs, ks = _as64(q_scale), _as64(k_scale)
    B, H, N, d = qv.shape
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    key_tile = np.arange(N) // tile_rows
    O = np.empty((B, H, len(rows), d))
    lse = np.empty((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            pos = 0
            for rr in _row_chunks(rows, N):
                dots = qv[b, h, rr] @ kv[b, h].T
                dequant = 1.0 / (qs[b, h, rr // tile_rows][:, None] * ks[b, h, key_tile][None, :])
                S = softmax_scale * dots * dequant
                if causal:
                    S = _causal_mask(S, rr)
                o, s = _softmax_rows(S, v[b, h])
                O[b, h, pos:pos + len(rr)] = o
                lse[b, h, pos:pos + len(rr)] = s
                pos += len(rr)
    return O, lse
