"""Pins of the float64 attention oracle against facts fixed outside it.

Each test checks the oracle against something other than its own formula:
brute-force scalar sums on tiny inputs, closed forms (zero queries or keys,
causal row 0, a single key, constant and affine V, a dominant key),
invariants (permutation of keys, probabilities summing to one with the
right log-ratios, the causal prefix property), the pages' block-by-block
online-softmax recurrences, and torch's own float64 softmax.  The last
test plants typical mistakes in a copy of the oracle and shows that the
pins catch every one of them.
"""
import importlib
import math

import numpy as np
import pytest

import oracle

oracle_attention_mod = importlib.import_module("oracle.attention")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --------------------------------------------------------------------------
# brute force: plain Python sums, no max subtraction, no numpy reductions
# --------------------------------------------------------------------------

def _brute(q, k, v, causal, scale):
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = range(i + 1) if causal else range(N)
                w = []
                for j in keys:
                    z = scale * math.fsum(q[b, h, i, c] * k[b, h, j, c] for c in range(d))
                    w.append(math.exp(z))
                tot = math.fsum(w)
                for c in range(d):
                    O[b, h, i, c] = math.fsum(wj * v[b, h, j, c] for wj, j in zip(w, keys)) / tot
                lse[b, h, i] = math.log(tot)
    return O, lse


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8, 17])
@pytest.mark.parametrize("d", [1, 2, 4, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(N, d, causal):
    shape = (1, 2, N, d)
    q, k, v = _rand(shape, 1), _rand(shape, 2), _rand(shape, 3)
    scale = 1.0 / math.sqrt(d)
    O, lse = oracle.attention(q, k, v, causal, scale)
    Ob, lseb = _brute(q, k, v, causal, scale)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lseb, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("which", ["q", "k"])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_operand_gives_prefix_mean(which, causal):
    shape = (2, 2, 37, 8)
    q, k, v = _rand(shape, 4), _rand(shape, 5), _rand(shape, 6)
    if which == "q":
        q[:] = 0.0
    else:
        k[:] = 0.0
    O, lse = oracle.attention(q, k, v, causal, 0.3)
    N = shape[2]
    counts = np.arange(1, N + 1) if causal else np.full(N, N)
    if causal:
        ref = np.cumsum(v, axis=2) / counts[None, None, :, None]
    else:
        ref = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(counts), lse.shape), rtol=1e-13, atol=1e-13)


def test_causal_row0_is_v0_and_lse_is_s00():
    shape = (3, 2, 20, 16)
    q, k, v = _rand(shape, 7), _rand(shape, 8), _rand(shape, 9)
    scale = 0.7
    O, lse = oracle.attention(q, k, v, True, scale)
    np.testing.assert_allclose(O[:, :, 0], v[:, :, 0], rtol=0, atol=1e-15)
    s00 = scale * np.einsum("bhc,bhc->bh", q[:, :, 0], k[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], s00, rtol=1e-13, atol=1e-13)


def test_single_key_returns_v():
    shape = (2, 3, 1, 5)
    q, k, v = _rand(shape, 10), _rand(shape, 11), _rand(shape, 12)
    for causal in (False, True):
        O, lse = oracle.attention(q, k, v, causal, 1.3)
        np.testing.assert_allclose(O, v, rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[..., 0], 1.3 * np.sum(q[..., 0, :] * k[..., 0, :], axis=-1), rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_and_affine_v(causal):
    shape = (1, 2, 29, 6)
    q, k, v = _rand(shape, 13, 2.0), _rand(shape, 14, 2.0), _rand(shape, 15)
    O_c, _ = oracle.attention(q, k, np.full(shape, -2.5), causal, 0.4)
    np.testing.assert_allclose(O_c, -2.5, rtol=1e-13)
    O, lse = oracle.attention(q, k, v, causal, 0.4)
    O_a, lse_a = oracle.attention(q, k, 3.0 * v - 1.25, causal, 0.4)
    np.testing.assert_allclose(O_a, 3.0 * O - 1.25, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(lse_a, lse)


def test_dominant_key_selects_its_value():
    N, d = 24, 8
    rng = np.random.default_rng(16)
    q = np.zeros((1, 1, N, d))
    q[..., 0] = 1.0
    k = rng.standard_normal((1, 1, N, d)) * 0.1
    k[..., 0] = 0.0
    j = 11
    k[0, 0, j, 0] = 60.0                       # logit 60 above every other key (scale 1)
    v = rng.standard_normal((1, 1, N, d))
    O, lse = oracle.attention(q, k, v, False, 1.0)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0, j], (N, d)), atol=N * math.exp(-59))
    np.testing.assert_allclose(lse[0, 0], 60.0, atol=N * math.exp(-59))


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_noncausal_key_permutation_invariance():
    shape = (2, 2, 33, 8)
    q, k, v = _rand(shape, 17), _rand(shape, 18), _rand(shape, 19)
    perm = np.random.default_rng(20).permutation(shape[2])
    O, lse = oracle.attention(q, k, v, False, 0.5)
    O_p, lse_p = oracle.attention(q, k[:, :, perm], v[:, :, perm], False, 0.5)
    np.testing.assert_allclose(O_p, O, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_p, lse, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_identity_v_exposes_probabilities(causal):
    """With V = I (d = N) the output rows are the softmax rows themselves."""
    N = 12
    q, k = _rand((1, 1, N, N), 21), _rand((1, 1, N, N), 22)
    v = np.eye(N)[None, None]
    scale = 0.6
    P, _ = oracle.attention(q, k, v, causal, scale)
    P = P[0, 0]
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(P >= 0)
    for i in range(N):
        allowed = list(range(i + 1)) if causal else list(range(N))
        if causal:
            assert np.all(P[i, i + 1:] == 0.0)
        a = allowed[0]
        for j in allowed[1:]:
            ds = scale * math.fsum(q[0, 0, i, c] * (k[0, 0, j, c] - k[0, 0, a, c]) for c in range(N))
            assert math.isclose(P[i, j] / P[i, a], math.exp(ds), rel_tol=1e-12)


def test_causal_prefix_property():
    shape = (1, 2, 40, 8)
    q, k, v = _rand(shape, 23), _rand(shape, 24), _rand(shape, 25)
    O, lse = oracle.attention(q, k, v, True, 0.35)
    for i in (0, 1, 7, 20, 39):
        s = slice(0, i + 1)
        O_nc, lse_nc = oracle.attention(q[:, :, s], k[:, :, s], v[:, :, s], False, 0.35)
        np.testing.assert_allclose(O[:, :, i], O_nc[:, :, i], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, i], lse_nc[:, :, i], rtol=1e-13, atol=1e-13)


def test_rows_subset_and_chunking(monkeypatch):
    shape = (2, 2, 70, 16)
    q, k, v = _rand(shape, 26), _rand(shape, 27), _rand(shape, 28)
    sel = np.array([0, 1, 31, 32, 63, 64, 69])
    for causal in (False, True):
        O, lse = oracle.attention(q, k, v, causal, 0.25)
        O_s, lse_s = oracle.attention(q, k, v, causal, 0.25, rows=sel)
        np.testing.assert_array_equal(O_s, O[:, :, sel])
        np.testing.assert_array_equal(lse_s, lse[:, :, sel])
        monkeypatch.setattr(oracle_attention_mod, "_CHUNK_ELEMS", 3 * 70)
        O_c, lse_c = oracle.attention(q, k, v, causal, 0.25)
        monkeypatch.undo()
        np.testing.assert_allclose(O_c, O, rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(lse_c, lse, rtol=1e-15, atol=1e-15)


def test_matches_torch_float64_softmax():
    torch = pytest.importorskip("torch")
    shape = (2, 3, 100, 16)
    q, k, v = _rand(shape, 29, 2.0), _rand(shape, 30, 2.0), _rand(shape, 31)
    scale = 1 / 4
    for causal in (False, True):
        O, lse = oracle.attention(q, k, v, causal, scale)
        tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
        s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) * scale
        if causal:
            s = s.masked_fill(torch.ones(100, 100, dtype=torch.bool).triu(1), float("-inf"))
        ref = torch.matmul(torch.softmax(s, dim=-1), tv)
        np.testing.assert_allclose(O, ref.numpy(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# the pages' online recurrences agree with the two-pass definition
# --------------------------------------------------------------------------

@pytest.mark.parametrize("block", [1, 3, 16, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrences_equal_two_pass(block, causal):
    N, d = 50, 8
    q, k, v = _rand((N, d), 32, 3.0), _rand((N, d), 33, 3.0), _rand((N, d), 34)
    O, lse = oracle.attention(q[None, None], k[None, None], v[None, None], causal, 0.5)
    for fn in (oracle.online_softmax_attention, oracle.online_softmax_eager):
        O_on, lse_on = fn(q, k, v, causal, 0.5, block)
        np.testing.assert_allclose(O_on, O[0, 0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse_on, lse[0, 0], rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# planted mistakes: each altered copy of the oracle must fail some pin
# --------------------------------------------------------------------------

def _mutant(kind):
    def attn(q, k, v, causal, scale):
        q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
        B, H, N, d = q.shape
        O = np.empty((B, H, N, d))
        lse = np.empty((B, H, N))
        for b in range(B):
            for h in range(H):
                sc = 1.0 if kind == "dropped_scale" else scale
                if kind == "transposed_scores":
                    S = sc * (k[b, h] @ q[b, h].T)
                else:
                    S = sc * (q[b, h] @ k[b, h].T)
                if causal:
                    i = np.arange(N)[:, None]
                    j = np.arange(N)[None, :]
                    drop = {"mask_flipped": j < i, "mask_strict": j >= i}.get(kind, j > i)
                    S = np.where(drop, -np.inf, S)
                axis = 0 if kind == "softmax_over_queries" else 1
                m = S.max(axis=axis, keepdims=True)
                e = np.exp(S - m)
                l = e.sum(axis=axis, keepdims=True)
                O[b, h] = (e / l) @ v[b, h]
                if kind == "lse_without_max":
                    lse[b, h] = np.log(e.sum(axis=1))
                else:
                    mr = S.max(axis=1)
                    lse[b, h] = mr + np.log(np.exp(S - mr[:, None]).sum(axis=1))
                    if kind == "lse_in_log2":
                        lse[b, h] /= np.log(2.0)
        return O, lse
    return attn


def _pins_pass(attn):
    """A compact run of the pins above against an arbitrary attention function."""
    try:
        for causal in (False, True):
            for N, d in ((5, 4), (8, 2)):
                shape = (1, 1, N, d)
                q, k, v = _rand(shape, 40 + N), _rand(shape, 50 + d), _rand(shape, 60)
                O, lse = attn(q, k, v, causal, 0.8)
                Ob, lseb = _brute(q, k, v, causal, 0.8)
                if not (np.allclose(O, Ob, rtol=1e-10, atol=1e-12) and np.allclose(lse, lseb, rtol=1e-10)):
                    return False
        return True
    except (FloatingPointError, ValueError):
        return False


def test_oracle_passes_compact_pins():
    assert _pins_pass(lambda q, k, v, c, s: oracle.attention(q, k, v, c, s))


@pytest.mark.parametrize("kind", ["dropped_scale", "transposed_scores", "mask_flipped", "mask_strict",
                                  "softmax_over_queries", "lse_without_max", "lse_in_log2"])
def test_planted_mistakes_are_caught(kind):
    with np.errstate(all="ignore"):
        assert not _pins_pass(_mutant(kind))
