"""GPU parity of the FP8 P*V forward (dtype FA_FP8_E4M3_PV) and its V
pre-pass, through the C ABI, against the float64 oracle.

The V pre-pass (fa_quant_v_pow2) must match oracle.quantize_v_pow2 bit for
bit (codes and block exponents).  The attention is compared with the oracle
on exactly the values the device uses for Q, K and V (decoded e4m3 with
their scales); what remains is the device's own e4m3 rounding of P, with a
power-of-two scale that puts each (query, tile) maximum in (224, 448]:
|dP| <= 2^-4 P in the normal range, so

    |O_gpu - O_ref| <= 2^-4 * A + 2^-8 |O_ref| + 5e-2,
    A = sum_j P_ij |V_jd| / l_i  (the oracle's attention with |V|),

the last term covering probabilities below the e4m3 normal range of their
tile and the fp32 dequantisation of the scores; lse is unaffected (l sums
the fp32 probabilities) and keeps the 1e-3 bound.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.fp8 import decode_e4m3, quantize_tiles
from parity_util import check_fp8pv as _check, oracle_fp8pv as _oracle_fp8pv, to_device
from tiled_attention_13_amd.inputs import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def _f8_slot(kk):
    return (((kk >> 2) & 1) << 5) | (((kk >> 5) & 1) << 4) | (((kk >> 3) & 3) << 2) | (kk & 3)


@pytest.mark.parametrize("N,d", [(1, 32), (63, 64), (200, 128), (1000, 64)])
def test_quant_v_bit_exact(gpu_lib, N, d):
    import torch
    from tiled_attention_13_amd import quant_v_pow2
    v = make_inputs(Workload("v", 2, 3, N, d, "bf16", False, 100 + N))[2]
    v[0, 0, :min(N, 64), 5] = 0.0                       # an all-zero column of a tile
    codes, sc = quant_v_pow2(to_device(v, "bf16"))
    torch.cuda.synchronize()
    codes = codes.cpu().numpy()
    sc = sc.cpu().numpy().astype(np.int64)
    ref_codes, ref_e = oracle.quantize_v_pow2(v)
    np.testing.assert_array_equal(sc, 127 - ref_e)
    n_tiles = (N + 63) // 64
    keys = np.arange(n_tiles * 64)
    pos = (keys // 64) * 64 + np.array([_f8_slot(k) for k in range(64)])[keys % 64]
    got = codes[:, :, :, pos[:N]].transpose(0, 1, 3, 2)    # back to [B, H, N, d]
    np.testing.assert_array_equal(got, ref_codes)
    assert np.all(codes[:, :, :, pos[N:]] == 0)


def _gpu(q, k, v, causal, scale):
    import torch
    from tiled_attention_13_amd import fwd
    tq, tk, tv = (to_device(a, "bf16") for a in (q, k, v))
    o, lse = fwd(tq, tk, tv, causal=causal, softmax_scale=scale, dtype="fp8pv")
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 200, 513])
def test_small_shapes(gpu_lib, d, causal, N):
    q, k, v = make_inputs(Workload("s", 1, 2, N, d, "bf16", False, 7000 + N + d))
    scale = 1.0 / math.sqrt(d)
    o, lse = _gpu(q, k, v, causal, scale)
    o_ref, lse_ref, a = _oracle_fp8pv(q, k, v, causal, scale)
    _check(o, lse, o_ref, lse_ref, a, f"fp8pv d={d} causal={causal} N={N}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", [(2, 8, 300), (3, 8, 700), (2, 24, 513)])
def test_d128_xcd_banded_order(gpu_lib, causal, B, H, N):
    """B*H a multiple of 8 with short heads: the 128-key kernel walks each XCD's
    heads in bands of 2, 3 and 6, with ragged query tiles; every (head, query
    tile) must be computed exactly once, so the whole output is compared."""
    q, k, v = make_inputs(Workload("band", B, H, N, 128, "bf16", False, 7100 + N + H))
    scale = 1.0 / math.sqrt(128)
    o, lse = _gpu(q, k, v, causal, scale)
    o_ref, lse_ref, a = _oracle_fp8pv(q, k, v, causal, scale)
    _check(o, lse, o_ref, lse_ref, a, f"fp8pv B={B} H={H} N={N} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [130, 257, 384, 640, 1000])
def test_d128_ring_wraparound(gpu_lib, causal, N):
    """The 128-key kernel's V ring holds two stages of e4m3 V^T rows plus the
    exponents of their two 64-key tiles: 2 to 8 key tiles, every stage reused for
    N >= 384, and last tiles holding one 64-key tile (130, 257) or a ragged one (1000)."""
    q, k, v = make_inputs(Workload("ring", 1, 2, N, 128, "bf16", False, 7200 + N))
    scale = 1.0 / math.sqrt(128)
    o, lse = _gpu(q, k, v, causal, scale)
    o_ref, lse_ref, a = _oracle_fp8pv(q, k, v, causal, scale)
    _check(o, lse, o_ref, lse_ref, a, f"fp8pv d=128 N={N} causal={causal}")


def test_closed_form_zero_queries(gpu_lib):
    """Q = 0: P is uniform over the visible keys, so O is the mean of the decoded V rows."""
    N, d = 300, 64
    q, k, v = make_inputs(Workload("s", 1, 2, N, d, "bf16", False, 71))
    q = np.zeros_like(q)
    o, lse = _gpu(q, k, v, True, 0.125)
    v8, ve = oracle.quantize_v_pow2(v)
    vd = oracle.dequantize_v_pow2(v8, ve)
    ref = np.cumsum(vd, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    # uniform P is 2^f * (1/...) -> exactly representable (a power of two), so only fp32 sums and bf16 output differ
    assert np.all(np.abs(o - ref) <= 1e-3 + 2.0 ** -8 * np.abs(ref))
    np.testing.assert_allclose(lse, np.log(np.arange(1, N + 1))[None, None, :].repeat(2, axis=1), atol=1e-5)


def test_full_size_sampled(gpu_lib):
    """The FP8 workload (1x16x32768x128, causal) with P*V on e4m3 too: sampled rows of two heads."""
    w = WORKLOADS["c5_fp8"]
    q, k, v = make_inputs(w)
    o, lse = _gpu(q, k, v, w.causal, w.softmax_scale)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, w.N - 1],
                                     np.random.default_rng(8).choice(w.N, 43, replace=False)]))
    for h in (0, w.H - 1):
        sl = slice(h, h + 1)
        o_ref, lse_ref, a = _oracle_fp8pv(q[:, sl], k[:, sl], v[:, sl], True, w.softmax_scale, rows=rows)
        _check(o[:, sl, rows], lse[:, sl, rows], o_ref, lse_ref, a, f"c5 fp8pv h={h}")
