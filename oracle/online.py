"""The pages' online-softmax recurrences, block by block (test infrastructure only).

These are not the oracle's definition (that is ``oracle.attention``); they
restate the tiled method the pages describe so that a test can show, in
float64, that streaming over key blocks gives the same O and lse as the
two-pass softmax over whole rows.

* ``online_softmax_attention`` -- the running max / running sum update of
  the Triton walkthrough's section 2.1, with the accumulator rescaled by the
  same factor and the division by the sum deferred to the end, as the
  "Flash Attention" tag page's excerpt on V2 describes (rescale postponed
  to the end).  Operators lost in the page text are read as
  ``m_new = max(rowmax(s), m)``, ``alpha = exp(m - m_new)``,
  ``beta = exp(s - m_new)``, ``l = alpha*l + rowsum(beta)``,
  ``acc = alpha*acc + beta @ V_block``.
* ``online_softmax_eager`` -- the FA1 form of "Core principles behind
  FlashAttention's speed-up", section 1.3: the output is kept normalised
  after every block (``out *= (d/new_d) exp(m - new_m)`` before adding the
  block's share).  The page loops over one query's keys; the reading taken
  is "for fixed query rows, iterate over key blocks", with its ``d`` being
  the running sum.

A block whose scores are all masked leaves the state unchanged.
"""
from __future__ import annotations

import numpy as np


def _block_scores(q, kb, scale, causal, rows, cols):
    s = scale * (q @ kb.T)
    if causal:
        s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
    return s


def online_softmax_attention(q, k, v, causal: bool, softmax_scale: float, block: int):
    """One (b, h) slice: q, k, v ``[N, d]`` float64 -> (O ``[N, d]``, lse ``[N]``)."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    N, d = q.shape
    rows = np.arange(N)
    m = np.full(N, -np.inf)
    l = np.zeros(N)
    acc = np.zeros((N, d))
    for j0 in range(0, k.shape[0], block):
        cols = np.arange(j0, min(j0 + block, k.shape[0]))
        s = _block_scores(q, k[cols], softmax_scale, causal, rows, cols)
        m_curr = np.maximum(s.max(axis=1), m)
        live = np.isfinite(m_curr)
        safe_m = np.where(live, m_curr, 0.0)
        alpha = np.where(live, np.exp(m - safe_m), 1.0)
        beta = np.exp(s - safe_m[:, None])          # exp(-inf) = 0 where masked
        l = alpha * l + beta.sum(axis=1)
        acc = alpha[:, None] * acc + beta @ v[cols]
        m = m_curr
    return acc / l[:, None], m + np.log(l)


def online_softmax_eager(q, k, v, causal: bool, softmax_scale: float, block: int):
    """FA1 eager-normalised recurrence for one (b, h) slice; same outputs."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    N, d = q.shape
    rows = np.arange(N)
    m = np.full(N, -np.inf)
    dsum = np.zeros(N)
    out = np.zeros((N, d))
    for j0 in range(0, k.shape[0], block):
        cols = np.arange(j0, min(j0 + block, k.shape[0]))
        s = _block_scores(q, k[cols], softmax_scale, causal, rows, cols)
        row_max = s.max(axis=1)
        has = np.isfinite(row_max)
        rm = np.where(has, row_max, 0.0)
        p_local = np.exp(s - rm[:, None])            # 0 where masked
        row_sum = p_local.sum(axis=1)
        new_m = np.maximum(m, row_max)
        nm = np.where(np.isfinite(new_m), new_m, 0.0)
        old_w = np.where(np.isfinite(m), np.exp(m - nm), 0.0)
        blk_w = np.where(has, np.exp(rm - nm), 0.0)
        new_d = dsum * old_w + row_sum * blk_w
        upd = new_d > 0
        nd = np.where(upd, new_d, 1.0)
        out = np.where(upd[:, None],
                       out * (dsum / nd * old_w)[:, None]
                       + (blk_w / nd)[:, None] * (p_local @ v[cols]),
                       out)
        m = np.where(upd, new_m, m)
        dsum = np.where(upd, new_d, dsum)
    return out, m + np.log(dsum)
