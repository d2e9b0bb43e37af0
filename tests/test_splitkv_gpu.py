"""GPU parity of attention over key ranges (fa_fwd_partial), the merge of
partial results (fa_merge) and split-KV attention (fa_fwd_splitkv), through
the C ABI, against the float64 oracle (oracle.splitkv and oracle.attention).

Tolerances: partial O is fp32 from bf16 products, compared like the bf16
forward (1e-2 + 2^-8 |ref|) and lse within 1e-3; merged and split-KV
outputs are bf16 and use the forward's bf16 rule.  The merge is also checked
alone on seeded synthetic partial results (host-generated, including empty
parts), where only fp32 arithmetic and the bf16 output rounding separate it
from the oracle.
"""
import math

import numpy as np
import pytest

import oracle
from parity_util import compare, to_device
from tiled_attention_13_amd.inputs import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def _inputs(B, H, N, d, seed, qk_gain=1.0):
    w = Workload("small", B, H, N, d, "bf16", False, seed, qk_gain=qk_gain)
    return make_inputs(w)


def _gpu_partial(q, k, v, lo, hi, causal, scale):
    import torch
    from tiled_attention_13_amd import fwd_partial
    tq, tk, tv = (to_device(a, "bf16") for a in (q, k, v))
    o, lse = fwd_partial(tq, tk, tv, lo, hi, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check_partial(o, lse, o_ref, lse_ref, what):
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), f"{what}: empty rows differ"
    empty = np.isneginf(lse_ref)
    assert np.all(o[empty] == 0.0), f"{what}: non-zero O on an empty row"
    fin = ~empty
    err = np.abs(o - o_ref)[fin]
    bound = 1e-2 + 2.0 ** -8 * np.abs(o_ref)[fin]
    assert np.all(err <= bound), f"{what}: max |dO| {err.max():.3g}"
    assert np.abs(lse[fin] - lse_ref[fin]).max(initial=0.0) <= 1e-3, what


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,lo,hi", [(300, 0, 300), (300, 64, 192), (300, 128, 300), (300, 256, 300),
                                     (300, 64, 64), (1000, 512, 1000), (65, 0, 64), (65, 64, 65)])
def test_partial_ranges(gpu_lib, d, causal, N, lo, hi):
    q, k, v = _inputs(1, 2, N, d, seed=4000 + N + lo + d)
    scale = 1.0 / math.sqrt(d)
    o, lse = _gpu_partial(q, k, v, lo, hi, causal, scale)
    o_ref, lse_ref = oracle.attention_partial(q, k, v, causal, scale, lo, hi)
    _check_partial(o, lse, o_ref, lse_ref, f"d={d} causal={causal} N={N} [{lo},{hi})")


@pytest.mark.parametrize("causal", [False, True])
def test_partials_merged_on_device_equal_attention(gpu_lib, causal):
    import torch
    from tiled_attention_13_amd import fwd_partial, merge
    N, d = 1000, 128
    q, k, v = _inputs(2, 2, N, d, seed=41, qk_gain=2.0)
    tq, tk, tv = (to_device(a, "bf16") for a in (q, k, v))
    cuts = [0, 128, 192, 640, 1000]
    parts = [fwd_partial(tq, tk, tv, lo, hi, causal=causal, softmax_scale=0.1) for lo, hi in zip(cuts[:-1], cuts[1:])]
    o, lse = merge(torch.stack([p[0] for p in parts]).contiguous(), torch.stack([p[1] for p in parts]).contiguous())
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, causal, 0.1)
    compare(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            o_ref, lse_ref, "bf16", f"merged partials causal={causal}")


def test_merge_on_synthetic_partials(gpu_lib):
    import torch
    from tiled_attention_13_amd import merge
    rng = np.random.default_rng(42)
    G, B, H, N, d = 5, 2, 3, 130, 64
    o_parts = rng.standard_normal((G, B, H, N, d)).astype(np.float32)
    lse_parts = (rng.standard_normal((G, B, H, N)) * 4).astype(np.float32)
    empty = rng.random((G, B, H, N)) < 0.3
    empty[:, 0, 0, 7] = True                       # a row that is empty in every part
    lse_parts[empty] = -np.inf
    o_parts[empty] = 0.0
    o, lse = merge(torch.from_numpy(o_parts).cuda(), torch.from_numpy(lse_parts).cuda())
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.merge_partials(o_parts, lse_parts)
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref))
    fin = np.isfinite(lse_ref)
    assert np.abs(lse[fin] - lse_ref[fin]).max() <= 1e-5 * max(1.0, np.abs(lse_ref[fin]).max())
    assert np.all(np.abs(o - o_ref) <= 1e-5 + 2.0 ** -8 * np.abs(o_ref))
    assert np.all(o[0, 0, 7] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,n_splits", [(1, 3), (65, 2), (300, 1), (300, 2), (300, 3), (1000, 4), (1000, 7),
                                        (200, 16)])
def test_splitkv_matches_attention(gpu_lib, causal, N, n_splits):
    import torch
    from tiled_attention_13_amd import fwd_splitkv
    d = 128
    q, k, v = _inputs(1, 3, N, d, seed=5000 + N + n_splits)
    tq, tk, tv = (to_device(a, "bf16") for a in (q, k, v))
    o, lse = fwd_splitkv(tq, tk, tv, n_splits, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, causal, 1 / math.sqrt(d))
    compare(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            o_ref, lse_ref, "bf16", f"splitkv N={N} splits={n_splits} causal={causal}")


def test_splitkv_full_size_sampled(gpu_lib):
    """The long causal workload's per-device share at eight devices (4 heads), 8 splits."""
    import torch
    from tiled_attention_13_amd import fwd_splitkv
    w = WORKLOADS["c4_bf16"]
    q, k, v = make_inputs(w, shape=(1, 4, w.N, w.d))
    tq, tk, tv = (to_device(a, "bf16") for a in (q, k, v))
    o, lse = fwd_splitkv(tq, tk, tv, 8, causal=True, softmax_scale=w.softmax_scale)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    rows = np.unique(np.concatenate([[0, 1, 2047, 2048, w.N - 1],
                                     np.random.default_rng(3).choice(w.N, 59, replace=False)]))
    for h in (0, 3):
        o_ref, lse_ref = oracle.attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], True, w.softmax_scale,
                                          rows=rows)
        compare(o[:, h:h + 1, rows], lse[:, h:h + 1, rows], o_ref, lse_ref, "bf16", f"splitkv c4 share h={h}")
