"""GPU parity of the attention backward (fa_bwd, through the C ABI) against
the float64 backward oracle.

The forward output and lse come from the device forward (fa_fwd) on the same
bf16 inputs, as a training step would use them.  Small shapes are compared
element by element and span several query and key tiles plus ragged tails;
the long workloads run at full size and are checked on sampled query rows
(dQ) and key columns (dK, dV) that the oracle computes one by one.

Tolerance (per element, per gradient tensor g of one (b, h) slice):
    |g_gpu - g_ref| <= BWD_TOL * max(max|g_ref|, G_FLOOR) + 2^-8 |g_ref|
The second term is the bf16 rounding of the output; the first covers the
bf16 rounding of P and dS before the matrix-core products (relative 2^-9
per term) and of the forward output O used for D = rowsum(dO * O).
G_FLOOR keeps the bound meaningful where the exact gradient vanishes (a
single key, a constant V): there dS is pure fp32 rounding, P*(dP - D) with
dP and D the same dot product summed in different orders.
"""
import math

import numpy as np
import pytest

import oracle
from parity_util import to_device
from tiled_attention_13_amd.inputs import WORKLOADS, Workload, make_grad, make_inputs

pytestmark = pytest.mark.gpu

BWD_TOL = 2e-2
G_FLOOR = 1e-3
U_BF16 = 2.0 ** -8


def _gpu_fwd_bwd(q, k, v, g, causal, scale):
    import torch
    from tiled_attention_13_amd import bwd, fwd
    tq, tk, tv, tg = (to_device(a, "bf16") for a in (q, k, v, g))
    o, lse = fwd(tq, tk, tv, causal=causal, softmax_scale=scale, dtype="bf16")
    dq, dk, dv = bwd(tq, tk, tv, o, tg, lse, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))


def _check(name, got, ref, what):
    assert np.all(np.isfinite(got)), f"{what} {name}: non-finite values"
    scale = np.abs(ref).max()
    err = np.abs(got - ref)
    bound = BWD_TOL * max(scale, G_FLOOR) + U_BF16 * np.abs(ref)
    if np.any(err > bound):
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what} {name}: {int(np.sum(err > bound))} elements out of bound; worst at {i}: "
                             f"gpu {got[i]:.6g} ref {ref[i]:.6g} (max|ref| {scale:.4g}, "
                             f"max err/max|ref| {err.max() / max(scale, 1e-300):.3g})")
    return float(err.max() / max(scale, 1e-300))


def _small(B, H, N, d, seed):
    w = Workload("small", B, H, N, d, "bf16", False, seed)
    q, k, v = make_inputs(w)
    return q, k, v, make_grad(w)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 129, 200, 300, 513])
def test_small_shapes_full_gradients(gpu_lib, d, causal, N):
    B, H = (2, 2) if N <= 129 else (1, 2)
    q, k, v, g = _small(B, H, N, d, seed=3000 + N + d)
    scale = 1.0 / math.sqrt(d)
    got = _gpu_fwd_bwd(q, k, v, g, causal, scale)
    ref = oracle.attention_backward(q, k, v, g, causal, scale)
    for b in range(B):
        for h in range(H):
            for name, a, r in zip(("dq", "dk", "dv"), got, ref):
                _check(name, a[b, h], r[b, h], f"d={d} causal={causal} N={N} b={b} h={h}")


def test_ragged_long_tail(gpu_lib):
    q, k, v, g = _small(1, 2, 1000, 64, seed=91)
    for causal in (False, True):
        got = _gpu_fwd_bwd(q, k, v, g, causal, 0.125)
        ref = oracle.attention_backward(q, k, v, g, causal, 0.125)
        for h in range(2):
            for name, a, r in zip(("dq", "dk", "dv"), got, ref):
                _check(name, a[0, h], r[0, h], f"N=1000 causal={causal} h={h}")


def test_closed_forms_on_device(gpu_lib):
    """N = 1 gives dQ = dK = 0 and dV = dO; a constant V gives dQ = dK = 0."""
    q, k, v, g = _small(2, 2, 1, 64, seed=5)
    dq, dk, dv = _gpu_fwd_bwd(q, k, v, g, True, 0.125)
    # P = exp(s - lse) is 1 up to fp32 rounding, which bf16 P absorbs
    assert np.abs(dq).max() < 1e-5 and np.abs(dk).max() < 1e-5
    np.testing.assert_array_equal(dv, g.astype(np.float64))
    q, k, v, g = _small(1, 2, 300, 64, seed=6)
    v = np.broadcast_to(v[:, :, :1, :], v.shape).copy()
    for causal in (False, True):
        dq, dk, dv = _gpu_fwd_bwd(q, k, v, g, causal, 0.125)
        # dS = P (dP - D) with dP_ij = D_i: zero up to the bf16 rounding of O in D
        assert np.abs(dq).max() < 1e-2 and np.abs(dk).max() < 1e-2


def test_column_sums_on_device(gpu_lib):
    """sum_j dV_j = sum_i dO_i (each P row sums to 1) at a size no oracle pass is needed for."""
    q, k, v, g = _small(1, 2, 2048, 128, seed=7)
    for causal in (False, True):
        dq, dk, dv = _gpu_fwd_bwd(q, k, v, g, causal, 1 / math.sqrt(128))
        ref = g.astype(np.float64).sum(axis=2)
        err = np.abs(dv.sum(axis=2) - ref)
        assert err.max() <= 2e-2 * np.abs(ref).max() + 0.05, err.max()


@pytest.mark.parametrize("name", ["c3_bf16", "c4_bf16"])
def test_workload_full_size_sampled(gpu_lib, name):
    w = WORKLOADS[name]
    q, k, v = make_inputs(w)
    g = make_grad(w)
    dq, dk, dv = _gpu_fwd_bwd(q, k, v, g, w.causal, w.softmax_scale)
    rng = np.random.default_rng(11)
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    for b, h in heads:
        rows = np.unique(np.concatenate([[0, 1, w.N - 1], rng.choice(w.N, 29, replace=False)]))
        ref_q = oracle.dq_rows(q, k, v, g, w.causal, w.softmax_scale, b, h, rows)
        ref_k, ref_v = oracle.dkdv_cols(q, k, v, g, w.causal, w.softmax_scale, b, h, rows)
        # the tolerance scale is the largest reference value of the sampled rows
        _check("dq", dq[b, h, rows], ref_q, f"{name} b={b} h={h}")
        _check("dk", dk[b, h, rows], ref_k, f"{name} b={b} h={h}")
        _check("dv", dv[b, h, rows], ref_v, f"{name} b={b} h={h}")
