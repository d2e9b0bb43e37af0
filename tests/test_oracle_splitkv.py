"""Pins of the partial-attention and merge oracle (oracle.splitkv).

Partial results are checked against plain Python sums over the key subset;
merged partials over any partition of the keys must reproduce the full
attention oracle (itself pinned in test_oracle.py); merging is invariant to
the order of the parts, a single part merges to itself and an empty part
(lse = -inf) changes nothing; rows that see no key of a range get O = 0 and
lse = -inf.  Planted mistakes in a copy of the merge or of the partial
attention fail these pins.
"""
import math

import numpy as np
import pytest

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _brute_partial(q, k, v, causal, scale, lo, hi):
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    lse = np.full((B, H, N), -math.inf)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = [j for j in range(lo, hi) if not (causal and j > i)]
                if not keys:
                    continue
                s = [scale * sum(q[b, h, i, t] * k[b, h, j, t] for t in range(d)) for j in keys]
                z = sum(math.exp(x) for x in s)
                lse[b, h, i] = math.log(z)
                for jj, j in enumerate(keys):
                    O[b, h, i] += math.exp(s[jj]) / z * v[b, h, j]
    return O, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lo,hi", [(0, 9), (3, 7), (5, 9), (8, 9), (4, 4)])
def test_partial_matches_brute_force(causal, lo, hi):
    shape = (1, 2, 9, 3)
    q, k, v = _rand(shape, 1, 2.0), _rand(shape, 2, 2.0), _rand(shape, 3)
    O, lse = oracle.attention_partial(q, k, v, causal, 0.6, lo, hi)
    Ob, lseb = _brute_partial(q, k, v, causal, 0.6, lo, hi)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-13)
    assert np.array_equal(np.isinf(lse), np.isinf(lseb))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], lseb[fin], rtol=1e-12)


def test_rows_seeing_no_key_are_empty():
    shape = (1, 1, 20, 4)
    q, k, v = _rand(shape, 4), _rand(shape, 5), _rand(shape, 6)
    O, lse = oracle.attention_partial(q, k, v, True, 0.5, 8, 16)
    assert np.all(O[0, 0, :8] == 0.0) and np.all(np.isneginf(lse[0, 0, :8]))
    assert np.all(np.isfinite(lse[0, 0, 8:]))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [(0, 70), (0, 1, 70), (0, 13, 14, 40, 70), (0, 35, 35, 70), (0, 64, 70)])
def test_merged_partials_equal_full_attention(causal, cuts):
    shape = (2, 2, 70, 8)
    q, k, v = _rand(shape, 7, 2.0), _rand(shape, 8, 2.0), _rand(shape, 9)
    parts = [oracle.attention_partial(q, k, v, causal, 0.4, lo, hi) for lo, hi in zip(cuts[:-1], cuts[1:])]
    O, lse = oracle.merge_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    Of, lsef = oracle.attention(q, k, v, causal, 0.4)
    np.testing.assert_allclose(O, Of, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lsef, rtol=1e-12, atol=1e-13)


def test_merge_identities():
    rng = np.random.default_rng(10)
    o = rng.standard_normal((3, 2, 5, 4))
    lse = rng.standard_normal((3, 2, 5)) * 3
    lse[1, 0, 2] = -np.inf
    o[1, 0, 2] = 0.0
    O, L = oracle.merge_partials(o, lse)
    perm = [2, 0, 1]
    O2, L2 = oracle.merge_partials(o[perm], lse[perm])
    np.testing.assert_allclose(O2, O, rtol=1e-14)
    np.testing.assert_allclose(L2, L, rtol=1e-14)
    O1, L1 = oracle.merge_partials(o[:1], lse[:1])
    np.testing.assert_allclose(O1, o[0], rtol=1e-15)
    np.testing.assert_allclose(L1, lse[0], rtol=1e-15)
    empty_o = np.zeros((1, 2, 5, 4))
    empty_l = np.full((1, 2, 5), -np.inf)
    Oe, Le = oracle.merge_partials(np.concatenate([o, empty_o]), np.concatenate([lse, empty_l]))
    np.testing.assert_allclose(Oe, O, rtol=1e-15)
    np.testing.assert_allclose(Le, L, rtol=1e-15)
    On, Ln = oracle.merge_partials(empty_o, empty_l)
    assert np.all(On == 0.0) and np.all(np.isneginf(Ln))


def test_split_ranges_partition_the_keys():
    for N in (1, 63, 64, 65, 1000, 16384):
        for n in (1, 2, 3, 4, 7):
            r = oracle.split_ranges(N, n)
            assert len(r) == n and r[0][0] == 0 and r[-1][1] == N
            assert all(a[1] == b[0] for a, b in zip(r[:-1], r[1:]))
            assert all((lo % 64 == 0 or lo == N) and lo <= hi for lo, hi in r)


# planted mistakes ---------------------------------------------------------

def _bad_merge_unnormalised(o, lse):
    w = np.exp(lse)
    return (w[..., None] * o).sum(axis=0), np.log(w.sum(axis=0))


def _bad_merge_plain_mean(o, lse):
    return o.mean(axis=0), np.log(np.exp(lse).sum(axis=0))


def _bad_partial_global_norm(q, k, v, causal, scale, lo, hi):
    # normalises over all keys instead of the range
    O, lse = oracle.attention(q, k, v, causal, scale)
    return O, lse


def _bad_partial_local_mask(q, k, v, causal, scale, lo, hi):
    # causal mask with key positions counted from the start of the range
    q2, k2, v2 = q, k[:, :, lo:hi], v[:, :, lo:hi]
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            S = scale * q2[b, h] @ k2[b, h].T
            if causal:
                S = np.where(np.arange(hi - lo)[None, :] > np.arange(N)[:, None], -np.inf, S)
            m = S.max(axis=1)
            e = np.exp(S - m[:, None])
            O[b, h] = (e / e.sum(axis=1, keepdims=True)) @ v2[b, h]
            lse[b, h] = m + np.log(e.sum(axis=1))
    return O, lse


def _pins_pass(partial, merge):
    shape = (1, 2, 30, 4)
    q, k, v = _rand(shape, 11, 2.0), _rand(shape, 12, 2.0), _rand(shape, 13)
    with np.errstate(all="ignore"):
        for causal in (False, True):
            cuts = (0, 10, 30)
            parts = [partial(q, k, v, causal, 0.5, lo, hi) for lo, hi in zip(cuts[:-1], cuts[1:])]
            O, lse = merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
            Of, lsef = oracle.attention(q, k, v, causal, 0.5)
            if not (np.allclose(O, Of, rtol=1e-10, atol=1e-12) and np.allclose(lse, lsef, rtol=1e-10)):
                return False
    return True


def test_oracle_passes_pins():
    assert _pins_pass(oracle.attention_partial, oracle.merge_partials)


@pytest.mark.parametrize("partial,merge", [
    (oracle.attention_partial, _bad_merge_unnormalised),
    (oracle.attention_partial, _bad_merge_plain_mean),
    (_bad_partial_global_norm, oracle.merge_partials),
    (_bad_partial_local_mask, oracle.merge_partials),
])
def test_planted_mistakes_are_caught(partial, merge):
    assert not _pins_pass(partial, merge)
