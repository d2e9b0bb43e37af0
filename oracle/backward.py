"""Attention backward by its definition, in float64 (test infrastructure only).

The forward pass is O = softmax(softmax_scale * Q K^T [causally masked]) V,
row by row (see ``oracle.attention``).  Given the gradient dO of some loss
with respect to O, the chain rule through the three steps gives, for every
(batch, head):

    P      = the softmax rows of the forward pass (masked entries are 0)
    dV     = P^T dO
    dP     = dO V^T
    D_i    = sum_j P[i, j] dP[i, j]
    dS     = P * (dP - D[:, None])      (softmax Jacobian, row by row)
    dQ     = softmax_scale * dS K
    dK     = softmax_scale * dS^T Q

A masked entry has P = 0, so it drops out of dV, dS, dQ and dK; D_i also
equals sum_k dO[i, k] O[i, k].

The pages state what the backward pass must not do rather than how it is
computed: the Triton walkthrough page (section 2.2) says the backward pass
recomputes intermediate results instead of storing them, and the tag page
(excerpt on V2) says V2 reassigns work between the forward and backward
passes.  The formulas above are the plain derivative of the forward
definition, which is what any such scheme computes up to rounding.

Everything is materialised row-chunk by row-chunk in float64 with numpy's
matmul as the only library primitive.  ``dq_rows`` and ``dkdv_cols`` give
the same quantities for a few query rows or key columns of one head, so
that large workloads can be checked on samples.
"""
from __future__ import annotations

import numpy as np

from .attention import _as64, _causal_mask, _row_chunks, attention, scores_rows


def _probs(q_rows, rows, k, causal, softmax_scale):
    """Softmax rows P[r, :] of the given query rows against every key."""
    S = scores_rows(q_rows, k, softmax_scale)
    if causal:
        S = _causal_mask(S, rows)
    m = S.max(axis=1, keepdims=True)
    e = np.exp(S - m)
    return e / e.sum(axis=1, keepdims=True)


def attention_backward(q, k, v, do, causal: bool, softmax_scale: float):
    """dQ, dK, dV of the attention forward for upstream gradient ``do``.

    All arrays ``[B, H, N, d]``; returns three float64 arrays of that shape.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, H, N, d = q.shape
    for a in (k, v, do):
        if a.shape != (B, H, N, d):
            raise ValueError("q, k, v, do must share the shape [B, H, N, d]")
    dq = np.zeros((B, H, N, d))
    dk = np.zeros((B, H, N, d))
    dv = np.zeros((B, H, N, d))
    all_rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            for rr in _row_chunks(all_rows, N):
                P = _probs(q[b, h, rr], rr, k[b, h], causal, softmax_scale)
                g = do[b, h, rr]
                dv[b, h] += P.T @ g
                dP = g @ v[b, h].T
                D = (P * dP).sum(axis=1)
                dS = P * (dP - D[:, None])
                dq[b, h, rr] = softmax_scale * (dS @ k[b, h])
                dk[b, h] += softmax_scale * (dS.T @ q[b, h, rr])
    return dq, dk, dv


def dq_rows(q, k, v, do, causal: bool, softmax_scale: float, b: int, h: int, rows):
    """dQ[b, h, rows] (float64 ``[R, d]``); each row needs only its own P and dP."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    rows = np.asarray(rows, dtype=np.int64)
    P = _probs(q[b, h, rows], rows, k[b, h], causal, softmax_scale)
    dP = do[b, h, rows] @ v[b, h].T
    D = (P * dP).sum(axis=1)
    dS = P * (dP - D[:, None])
    return softmax_scale * (dS @ k[b, h])


def dkdv_cols(q, k, v, do, causal: bool, softmax_scale: float, b: int, h: int, cols):
    """dK[b, h, cols] and dV[b, h, cols] (float64 ``[C, d]`` each).

    A key column needs the probabilities of every query row against it, so
    the row statistics (lse and D) of the whole head are computed first
    from the forward definition, in row chunks; then, for the sampled keys
    only, P[i, j] = exp(S[i, j] - lse_i), dP[i, j] = dO_i . V_j and
    dS[i, j] = P[i, j] (dP[i, j] - D_i).
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    N = q.shape[2]
    cols = np.asarray(cols, dtype=np.int64)
    O, lse = attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], causal, softmax_scale)
    O, lse = O[0, 0], lse[0, 0]
    D = (do[b, h] * O).sum(axis=1)                          # D_i = sum_k dO_ik O_ik
    S = softmax_scale * (q[b, h] @ k[b, h, cols].T)         # [N, C]
    if causal:
        S = np.where(cols[None, :] > np.arange(N)[:, None], -np.inf, S)
    P = np.exp(S - lse[:, None])
    dP = do[b, h] @ v[b, h, cols].T
    dS = P * (dP - D[:, None])
    dv = P.T @ do[b, h]
    dk = softmax_scale * (dS.T @ q[b, h])
    return dk, dv
