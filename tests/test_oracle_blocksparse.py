"""Pins of the block-sparse attention oracle (oracle.blocksparse).

An all-ones table reproduces the dense oracle; a block-diagonal table equals
dense attention run on every 64-row sub-sequence on its own; a table with a
single allowed key-block column equals the partial-attention oracle over
that key range; plain Python sums agree on a small ragged case; rows whose
blocks are all masked are empty; the visible-pair count has closed forms.
Planted mistakes (a transposed table, a wrong block size, the causal mask
dropped) fail these pins.
"""
import math

import numpy as np
import pytest

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_is_dense(causal):
    shape = (2, 2, 150, 8)
    q, k, v = _rand(shape, 1, 2.0), _rand(shape, 2, 2.0), _rand(shape, 3)
    nb = 3
    O, lse = oracle.attention_blocksparse(q, k, v, np.ones((nb, nb), np.uint8), causal, 0.4)
    Od, lsed = oracle.attention(q, k, v, causal, 0.4)
    np.testing.assert_allclose(O, Od, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lsed, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_block_diagonal_is_independent_subsequences(causal):
    N = 200
    shape = (1, 2, N, 8)
    q, k, v = _rand(shape, 4, 2.0), _rand(shape, 5, 2.0), _rand(shape, 6)
    nb = 4
    O, lse = oracle.attention_blocksparse(q, k, v, np.eye(nb, dtype=np.uint8), causal, 0.3)
    for bi in range(nb):
        s = slice(64 * bi, min(N, 64 * bi + 64))
        Ob, lseb = oracle.attention(q[:, :, s], k[:, :, s], v[:, :, s], causal, 0.3)
        np.testing.assert_allclose(O[:, :, s], Ob, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, s], lseb, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_single_key_column_is_partial_attention(causal):
    N = 200
    shape = (1, 2, N, 8)
    q, k, v = _rand(shape, 7, 2.0), _rand(shape, 8, 2.0), _rand(shape, 9)
    m = np.zeros((4, 4), np.uint8)
    m[:, 2] = 1
    O, lse = oracle.attention_blocksparse(q, k, v, m, causal, 0.3)
    Op, lsep = oracle.attention_partial(q, k, v, causal, 0.3, 128, 192)
    np.testing.assert_allclose(O, Op, rtol=1e-12, atol=1e-13)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lsep))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], lsep[fin], rtol=1e-12)


def test_matches_brute_force_ragged():
    N, d = 130, 3
    shape = (1, 1, N, d)
    q, k, v = _rand(shape, 10, 2.0), _rand(shape, 11, 2.0), _rand(shape, 12)
    m = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 0]], np.uint8)
    for causal in (False, True):
        O, lse = oracle.attention_blocksparse(q, k, v, m, causal, 0.7)
        for i in range(N):
            keys = [j for j in range(N) if m[i // 64, j // 64] and not (causal and j > i)]
            if not keys:
                assert np.all(O[0, 0, i] == 0) and np.isneginf(lse[0, 0, i])
                continue
            s = [0.7 * sum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d)) for j in keys]
            z = sum(math.exp(x) for x in s)
            ref = sum(math.exp(x) / z * v[0, 0, j] for x, j in zip(s, keys))
            np.testing.assert_allclose(O[0, 0, i], ref, rtol=1e-12, atol=1e-13)
            assert abs(lse[0, 0, i] - math.log(z)) < 1e-12 * max(1.0, abs(math.log(z)))


def test_per_head_tables_and_empty_rows():
    N = 128
    shape = (1, 2, N, 4)
    q, k, v = _rand(shape, 13), _rand(shape, 14), _rand(shape, 15)
    m = np.zeros((1, 2, 2, 2), np.uint8)
    m[0, 0] = [[1, 0], [0, 0]]           # head 0: rows 64.. see nothing
    m[0, 1] = [[0, 0], [1, 1]]           # head 1: rows 0..63 see nothing
    O, lse = oracle.attention_blocksparse(q, k, v, m, False, 0.5)
    assert np.all(O[0, 0, 64:] == 0) and np.all(np.isneginf(lse[0, 0, 64:]))
    assert np.all(O[0, 1, :64] == 0) and np.all(np.isneginf(lse[0, 1, :64]))
    Od, lsed = oracle.attention(q[:, :1, :64], k[:, :1, :64], v[:, :1, :64], False, 0.5)
    np.testing.assert_allclose(O[:, :1, :64], Od, rtol=1e-12)


def test_visible_pairs_closed_forms():
    for N in (1, 64, 100, 200):
        nb = -(-N // 64)
        ones = np.ones((nb, nb), np.uint8)
        assert oracle.visible_pairs(ones, N, False) == N * N
        assert oracle.visible_pairs(ones, N, True) == N * (N + 1) // 2
        sizes = [min(64, N - 64 * b) for b in range(nb)]
        assert oracle.visible_pairs(np.eye(nb, dtype=np.uint8), N, False) == sum(s * s for s in sizes)


def _pins_pass(fn):
    N = 200
    shape = (1, 1, N, 4)
    q, k, v = _rand(shape, 16, 2.0), _rand(shape, 17, 2.0), _rand(shape, 18)
    eye = np.eye(4, dtype=np.uint8)
    col = np.zeros((4, 4), np.uint8)
    col[:, 1] = 1
    col[3, 0] = 1
    with np.errstate(all="ignore"):
        for causal in (False, True):
            O, lse = fn(q, k, v, eye, causal, 0.3)
            for bi in range(4):
                s = slice(64 * bi, min(N, 64 * bi + 64))
                Ob, _ = oracle.attention(q[:, :, s], k[:, :, s], v[:, :, s], causal, 0.3)
                if not np.allclose(O[:, :, s], Ob, rtol=1e-10, atol=1e-12):
                    return False
            O, lse = fn(q, k, v, col, causal, 0.3)
            Ob, lseb = oracle.attention_blocksparse(q, k, v, col, causal, 0.3)
            if not np.allclose(O, Ob, rtol=1e-10, atol=1e-12):
                return False
    return True


def _mutant(kind):
    def fn(q, k, v, m, causal, scale):
        if kind == "transposed":
            return oracle.attention_blocksparse(q, k, v, np.asarray(m).T, causal, scale)
        if kind == "no_causal":
            return oracle.attention_blocksparse(q, k, v, m, False, scale)
        # block size 32: every 64-block entry covers a 32x32 block instead
        N = q.shape[2]
        nb32 = -(-N // 32)
        idx = np.minimum(np.arange(nb32), np.asarray(m).shape[0] - 1)
        m32 = np.asarray(m)[idx[:, None], idx[None, :]]
        allow = m32[(np.arange(N) // 32)[:, None], (np.arange(N) // 32)[None, :]] != 0
        nb = -(-N // 64)
        big = np.zeros((nb, nb), np.uint8)
        Oout = np.zeros(q.shape)
        lout = np.full(q.shape[:3], -np.inf)
        for i in range(N):
            vis = allow[i] & ((np.arange(N) <= i) if causal else True)
            if not vis.any():
                continue
            s = scale * (q[0, 0, i] @ k[0, 0].T)
            s = np.where(vis, s, -np.inf)
            e = np.exp(s - s.max())
            Oout[0, 0, i] = e @ v[0, 0] / e.sum()
            lout[0, 0, i] = s.max() + np.log(e.sum())
        return Oout, lout
    return fn


def test_oracle_passes_pins():
    assert _pins_pass(oracle.attention_blocksparse)


@pytest.mark.parametrize("kind", ["transposed", "no_causal", "block32"])
def test_planted_mistakes_are_caught(kind):
    assert not _pins_pass(_mutant(kind))
