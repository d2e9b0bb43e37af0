"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle on
the same seeded inputs, compare within the stated tolerances.

Tolerance rule (per element, O):  |O_gpu - O_ref| <= tol + u * |O_ref|
with tol = 1e-4 (fp32), 1e-2 (bf16), 5e-2 (fp8) and u the unit roundoff of
the output type (2^-24 for fp32 output, 2^-8 for bf16 output): the output
itself is rounded to that type, and for |O| >= 4 one bf16 rounding step
alone exceeds 1e-2.  lse: |lse_gpu - lse_ref| <= 1e-3 absolute.
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle.fp8 import decode_e4m3, quantize_tiles

TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 5e-2}
UNIT = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8, "fp8": 2.0 ** -8}
LSE_TOL = 1e-3


def to_device(arr, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr)).to("cuda")
    return t if dtype == "f32" else t.to(torch.bfloat16)


def gpu_forward(q, k, v, dtype, causal, scale):
    """Run fa_fwd on host arrays; returns (O float64, lse float64) on the host."""
    import torch
    from tiled_attention_13_amd import fwd
    tq, tk, tv = (to_device(a, dtype) for a in (q, k, v))
    o, lse = fwd(tq, tk, tv, causal=causal, softmax_scale=scale, dtype=dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle_forward(q, k, v, dtype, causal, scale, rows=None):
    """The oracle on exactly the values the device receives (fp8: its own quantisation)."""
    if dtype == "fp8":
        q8, qs = quantize_tiles(q)
        k8, ks = quantize_tiles(k)
        return oracle.attention_fp8(decode_e4m3(q8), qs, decode_e4m3(k8), ks, v, causal, scale, rows=rows)
    return oracle.attention(q, k, v, causal, scale, rows=rows)


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what="", lse_tol=LSE_TOL):
    """Assert the tolerance rule; return a small report dict."""
    tol, u = TOL[dtype], UNIT[dtype]
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    assert np.all(np.isfinite(lse_gpu)), f"{what}: non-finite lse"
    err = np.abs(o_gpu - o_ref)
    bound = tol + u * np.abs(o_ref)
    over = err > bound
    lse_err = np.abs(lse_gpu - lse_ref)
    rep = {"max_abs_dO": float(err.max()), "n_raw_over_tol": int(np.sum(err > tol)),
           "n_over_bound": int(over.sum()), "max_abs_dlse": float(lse_err.max())}
    if over.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {rep['n_over_bound']} elements outside tol {tol} + {u}|ref|; "
                             f"worst at {idx}: gpu {o_gpu[idx]!r} ref {o_ref[idx]!r}; {rep}")
    assert lse_err.max() <= lse_tol, f"{what}: lse error {lse_err.max()} > {lse_tol}; {rep}"
    return rep


def sample_rows(N, seed, n_random=24, qtile=256):
    """Query rows to check at full size: ends, the edges of a wave's 32 rows,
    of a 64-row block and of the kernel's 256-row query tile, and random rows."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 31, 32, 63, 64, 127, 128, qtile - 1, qtile, qtile + 1, N // 2 - 1, N // 2,
             N - qtile - 1, N - qtile, N - qtile + 1, N - 129, N - 128,
             N - 65, N - 64, N - 33, N - 32, N - 2, N - 1]
    rows = np.concatenate([np.array(fixed), rng.choice(N, n_random, replace=False)])
    rows = rows[(rows >= 0) & (rows < N)]
    return np.unique(rows)


def oracle_fp8pv(q, k, v, causal, scale, rows=None):
    """The oracle on the decoded e4m3 Q, K (per-tile scales) and V (power-of-two
    scales), and the attention of |V| that bounds the effect of rounding P."""
    q8, qs = quantize_tiles(q)
    k8, ks = quantize_tiles(k)
    v8, ve = oracle.quantize_v_pow2(v)
    vd = oracle.dequantize_v_pow2(v8, ve)
    qd, kd = decode_e4m3(q8), decode_e4m3(k8)
    o, lse = oracle.attention_fp8(qd, qs, kd, ks, vd, causal, scale, rows=rows)
    a, _ = oracle.attention_fp8(qd, qs, kd, ks, np.abs(vd), causal, scale, rows=rows)
    return o, lse, a


def check_fp8pv(o, lse, o_ref, lse_ref, a, what, lse_tol=LSE_TOL):
    """|O - O_ref| <= 2^-4 A + 2^-8 |O_ref| + 5e-2 (A: attention of |V|); lse within lse_tol."""
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what
    err = np.abs(o - o_ref)
    bound = 2.0 ** -4 * a + 2.0 ** -8 * np.abs(o_ref) + 5e-2
    if np.any(err > bound):
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int((err > bound).sum())} elements out of bound; worst {i}: gpu {o[i]:.5g} "
                             f"ref {o_ref[i]:.5g} bound {bound[i]:.3g}")
    assert np.abs(lse - lse_ref).max() <= lse_tol, what
    return float(err.max())
