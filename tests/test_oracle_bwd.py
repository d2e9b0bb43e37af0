"""Pins of the float64 attention-backward oracle against facts fixed outside it.

The gradients are checked against central finite differences of the forward
oracle (itself pinned in test_oracle.py), against torch autograd in float64
on the CPU, against closed forms (a single key, constant V, zero queries)
and invariants (the columns of dK sum to zero, the columns of dV sum to the
columns of dO).  The sampled-row and sampled-column helpers must agree with
the full computation.  The last test plants typical mistakes in a copy of
the backward and shows that the finite-difference pin catches each one.
"""
import numpy as np
import pytest

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _loss(q, k, v, g, causal, scale):
    O, _ = oracle.attention(q, k, v, causal, scale)
    return float((O * g).sum())


def _fd_grads(q, k, v, g, causal, scale, eps=1e-6):
    """Central differences of L = sum(O * g) with respect to q, k and v."""
    out = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        grad = np.zeros_like(args[which])
        it = np.nditer(args[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            x0 = args[which][idx]
            args[which][idx] = x0 + eps
            lp = _loss(*args, g, causal, scale)
            args[which][idx] = x0 - eps
            lm = _loss(*args, g, causal, scale)
            args[which][idx] = x0
            grad[idx] = (lp - lm) / (2 * eps)
        out.append(grad)
    return out


@pytest.mark.parametrize("N,d", [(1, 3), (5, 4), (9, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_finite_differences(N, d, causal):
    shape = (1, 2, N, d)
    q, k, v, g = _rand(shape, 1 + N), _rand(shape, 2 + d), _rand(shape, 3), _rand(shape, 4)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, causal, 0.7)
    fq, fk, fv = _fd_grads(q, k, v, g, causal, 0.7)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd_float64(causal):
    torch = pytest.importorskip("torch")
    shape = (2, 3, 70, 16)
    q, k, v, g = _rand(shape, 11, 2.0), _rand(shape, 12, 2.0), _rand(shape, 13), _rand(shape, 14)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    S = 0.25 * tq @ tk.transpose(-1, -2)
    if causal:
        S = S.masked_fill(torch.ones(70, 70, dtype=torch.bool).triu(1), float("-inf"))
    O = torch.softmax(S, dim=-1) @ tv
    O.backward(torch.tensor(g, dtype=torch.float64))
    dq, dk, dv = oracle.attention_backward(q, k, v, g, causal, 0.25)
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_single_key():
    # N = 1: O = V whatever Q and K are, so dQ = dK = 0 and dV = dO
    shape = (2, 2, 1, 5)
    q, k, v, g = _rand(shape, 21), _rand(shape, 22), _rand(shape, 23), _rand(shape, 24)
    for causal in (False, True):
        dq, dk, dv = oracle.attention_backward(q, k, v, g, causal, 1.3)
        assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
        np.testing.assert_allclose(dv, g, rtol=1e-15, atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_has_no_score_gradient(causal):
    # every row of V equal: O does not depend on P, so dQ = dK = 0
    shape = (1, 2, 12, 4)
    q, k, g = _rand(shape, 31, 2.0), _rand(shape, 32, 2.0), _rand(shape, 33)
    v = np.broadcast_to(_rand((1, 2, 1, 4), 34), shape).copy()
    dq, dk, dv = oracle.attention_backward(q, k, v, g, causal, 0.9)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_closed_form(causal):
    # Q = 0: every allowed key gets weight 1/n_i (n_i = N, or i + 1 causal), so
    #   dV_j = sum_{i: j allowed} dO_i / n_i
    #   dQ_i = scale/n_i * sum_{j allowed} (dO_i . (V_j - mean_i V)) K_j
    #   dK   = 0 (dK_j = scale * sum_i dS_ij Q_i with Q = 0)
    N, d, scale = 10, 3, 0.6
    shape = (1, 1, N, d)
    q = np.zeros(shape)
    k, v, g = _rand(shape, 41), _rand(shape, 42), _rand(shape, 43)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, causal, scale)
    K, V, G = k[0, 0], v[0, 0], g[0, 0]
    ref_dv = np.zeros((N, d))
    ref_dq = np.zeros((N, d))
    for i in range(N):
        n = i + 1 if causal else N
        vbar = V[:n].mean(axis=0)
        for j in range(n):
            ref_dv[j] += G[i] / n
            ref_dq[i] += scale / n * float(G[i] @ (V[j] - vbar)) * K[j]
    np.testing.assert_allclose(dv[0, 0], ref_dv, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dq[0, 0], ref_dq, rtol=1e-12, atol=1e-14)
    assert np.abs(dk).max() == 0.0


@pytest.mark.parametrize("causal", [False, True])
def test_column_sum_invariants(causal):
    # each softmax row sums to 1 (so sum_j dV_j = sum_i dO_i) and each dS row
    # sums to 0 (so sum_j dK_j = 0)
    shape = (2, 2, 33, 8)
    q, k, v, g = _rand(shape, 51, 2.0), _rand(shape, 52, 2.0), _rand(shape, 53), _rand(shape, 54)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, causal, 0.5)
    np.testing.assert_allclose(dv.sum(axis=2), g.sum(axis=2), rtol=1e-12, atol=1e-12)
    assert np.abs(dk.sum(axis=2)).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_helpers_match_full(causal):
    shape = (2, 3, 40, 8)
    q, k, v, g = _rand(shape, 61, 2.0), _rand(shape, 62, 2.0), _rand(shape, 63), _rand(shape, 64)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, causal, 0.4)
    rows = np.array([0, 7, 39])
    cols = np.array([0, 13, 38, 39])
    np.testing.assert_allclose(oracle.dq_rows(q, k, v, g, causal, 0.4, 1, 2, rows), dq[1, 2, rows],
                               rtol=1e-12, atol=1e-14)
    sk, sv = oracle.dkdv_cols(q, k, v, g, causal, 0.4, 1, 2, cols)
    np.testing.assert_allclose(sk, dk[1, 2, cols], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(sv, dv[1, 2, cols], rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------
# planted mistakes: each altered copy of the backward must fail the FD pin
# --------------------------------------------------------------------------

def _mutant(kind):
    def bwd(q, k, v, g, causal, scale):
        B, H, N, d = q.shape
        dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
        for b in range(B):
            for h in range(H):
                S = scale * q[b, h] @ k[b, h].T
                if causal:
                    S = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, S)
                P = np.exp(S - S.max(axis=1, keepdims=True))
                P /= P.sum(axis=1, keepdims=True)
                dP = g[b, h] @ v[b, h].T
                D = dP.sum(axis=1) if kind == "unweighted_D" else (P * dP).sum(axis=1)
                dS = P * dP if kind == "no_D_term" else P * (dP - D[:, None])
                dv[b, h] = P @ g[b, h] if kind == "dv_untransposed" else P.T @ g[b, h]
                dq[b, h] = scale * dS @ k[b, h]
                dk_s = 1.0 if kind == "dk_without_scale" else scale
                dk[b, h] = dk_s * (dS @ q[b, h] if kind == "dk_untransposed" else dS.T @ q[b, h])
        return dq, dk, dv
    return bwd


def _fd_pin_passes(bwd):
    for causal in (False, True):
        shape = (1, 1, 6, 3)
        q, k, v, g = _rand(shape, 71), _rand(shape, 72), _rand(shape, 73), _rand(shape, 74)
        got = bwd(q, k, v, g, causal, 0.7)
        ref = _fd_grads(q, k, v, g, causal, 0.7)
        if not all(np.allclose(a, b, rtol=1e-6, atol=1e-8) for a, b in zip(got, ref)):
            return False
    return True


def test_oracle_passes_fd_pin():
    assert _fd_pin_passes(oracle.attention_backward)


@pytest.mark.parametrize("kind", ["unweighted_D", "no_D_term", "dv_untransposed", "dk_without_scale",
                                  "dk_untransposed"])
def test_planted_mistakes_are_caught(kind):
    assert not _fd_pin_passes(_mutant(kind))
