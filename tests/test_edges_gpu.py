"""Edge cases of the forward and backward through the C ABI against the
float64 oracle: extreme softmax scales (near-uniform and near-one-hot rows,
which stress the lazy reference max and the fp8 scales) and a very long
single head (large offsets inside one (b, h) slice), checked on sampled rows
with the same tolerance rules as the other parity tests."""
import math

import numpy as np
import pytest

import oracle
from parity_util import compare, gpu_forward, oracle_forward, to_device
from tiled_attention_13_amd.inputs import Workload, make_grad, make_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("scale", [1e-3, 0.5, 3.0])
@pytest.mark.parametrize("causal", [False, True])
def test_extreme_softmax_scales(gpu_lib, dtype, scale, causal):
    q, k, v = make_inputs(Workload("e", 1, 2, 700, 64, dtype, False, 90))
    o, lse = gpu_forward(q, k, v, dtype, causal, scale)
    o_ref, lse_ref = oracle_forward(q, k, v, dtype, causal, scale)
    # the e4m3 MFMA adds each run of 8 products aligned to the largest with
    # about 14 bits (tests/test_fp8_accumulation_gpu.py), so with logits near
    # 70 lse is only good to that relative precision; bf16 and fp32 keep the
    # absolute 1e-3
    lse_tol = 1e-3 + (2.0 ** -13 * np.abs(lse_ref).max() if dtype == "fp8" else 0.0)
    compare(o, lse, o_ref, lse_ref, dtype, f"{dtype} scale={scale} causal={causal}", lse_tol=lse_tol)


def _jump_inputs(N, d, seed):
    """Q and K share a direction u: keys of the first half score about 0, keys of
    the second half about 40 (58 in base-2 units), so every query that sees the
    second half moves its reference max by more than the kernels' lazy-rescale
    slack of 45 (base-2) and rescales its partial O by a factor in (0, 1)."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = 0.3 * rng.standard_normal((1, 2, N, d)) + 21.3 * u
    k = 0.3 * rng.standard_normal((1, 2, N, d))
    k[:, :, N // 2:] += 21.3 * u
    v = rng.standard_normal((1, 2, N, d))
    bf = lambda a: np.asarray(torch_bf16_round(a.astype(np.float32)), dtype=np.float32)
    return bf(q), bf(k), bf(v)


def torch_bf16_round(a):
    import torch
    return torch.from_numpy(a).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp8pv"])
@pytest.mark.parametrize("causal", [False, True])
def test_forced_rescale_d128(gpu_lib, dtype, causal):
    """d = 128 (the LDS-DMA kernels of the headline, FP8 and FP8 P*V paths) with a
    score jump that forces the O rescale; the jump is checked on the inputs."""
    from parity_util import check_fp8pv, oracle_fp8pv
    N, d = 1024, 128
    scale = 1.0 / math.sqrt(d)
    q, k, v = _jump_inputs(N, d, 96)
    s = scale * np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64))
    first, second = s[..., : N // 2].max(axis=-1), s[..., N // 2:].max(axis=-1)
    assert np.all((second - first) * math.log2(math.e) > 45.0), "inputs do not force a rescale"
    assert np.all(second < 60.0)
    o, lse = gpu_forward(q, k, v, dtype, causal, scale)
    if dtype == "fp8pv":
        o_ref, lse_ref, a = oracle_fp8pv(q, k, v, causal, scale)
        check_fp8pv(o, lse, o_ref, lse_ref, a, f"fp8pv rescale causal={causal}",
                    lse_tol=1e-3 + 2.0 ** -13 * np.abs(lse_ref).max())
        return
    o_ref, lse_ref = oracle_forward(q, k, v, dtype, causal, scale)
    lse_tol = 1e-3 + (2.0 ** -13 * np.abs(lse_ref).max() if dtype == "fp8" else 0.0)
    compare(o, lse, o_ref, lse_ref, dtype, f"{dtype} rescale causal={causal}", lse_tol=lse_tol)


@pytest.mark.parametrize("causal", [False, True])
def test_forced_rescale_d32(gpu_lib, causal):
    """bf16 d = 32 (its own kernel, whose softmax first tries the current reference
    without the row max): the score jump makes every query that sees the second
    half take the full step and rescale O."""
    N, d = 1024, 32
    q, k, v = _jump_inputs(N, d, 97)
    scale = 40.0 / 21.3 ** 2                         # the jump is ~40 in natural units, as at d = 128
    s = scale * np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64))
    first, second = s[..., : N // 2].max(axis=-1), s[..., N // 2:].max(axis=-1)
    assert np.all((second - first) * math.log2(math.e) > 45.0), "inputs do not force a rescale"
    assert np.all(second < 60.0)
    o, lse = gpu_forward(q, k, v, "bf16", causal, scale)
    o_ref, lse_ref = oracle_forward(q, k, v, "bf16", causal, scale)
    compare(o, lse, o_ref, lse_ref, "bf16", f"d=32 rescale causal={causal}")


def test_long_single_head_forward(gpu_lib):
    """B = H = 1, N = 262144, d = 64, causal: offsets up to 32 MiB inside one slice."""
    w = Workload("long", 1, 1, 262144, 64, "bf16", True, 91)
    q, k, v = make_inputs(w)
    o, lse = gpu_forward(q, k, v, "bf16", True, 0.125)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, w.N // 2, w.N - 1],
                                     np.random.default_rng(9).choice(w.N, 26, replace=False)]))
    o_ref, lse_ref = oracle.attention(q, k, v, True, 0.125, rows=rows)
    compare(o[:, :, rows], lse[:, :, rows], o_ref, lse_ref, "bf16", "N=262144")


def test_long_single_head_backward(gpu_lib):
    import torch
    from tiled_attention_13_amd import bwd, fwd
    w = Workload("longb", 1, 1, 32768, 64, "bf16", True, 92)
    q, k, v = make_inputs(w)
    g = make_grad(w)
    tq, tk, tv, tg = (to_device(a, "bf16") for a in (q, k, v, g))
    o, lse = fwd(tq, tk, tv, causal=True, softmax_scale=0.125)
    dq, dk, dv = bwd(tq, tk, tv, o, tg, lse, causal=True, softmax_scale=0.125)
    torch.cuda.synchronize()
    dq, dk, dv = (t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))
    rows = np.unique(np.concatenate([[0, 127, 128, w.N - 1], np.random.default_rng(10).choice(w.N, 20, replace=False)]))
    ref_q = oracle.dq_rows(q, k, v, g, True, 0.125, 0, 0, rows)
    ref_k, ref_v = oracle.dkdv_cols(q, k, v, g, True, 0.125, 0, 0, rows)
    for name, got, ref in (("dq", dq[0, 0, rows], ref_q), ("dk", dk[0, 0, rows], ref_k), ("dv", dv[0, 0, rows], ref_v)):
        err = np.abs(got - ref)
        bound = 2e-2 * max(np.abs(ref).max(), 1e-3) + 2.0 ** -8 * np.abs(ref)
        assert np.all(err <= bound), (name, float(err.max()), float(np.abs(ref).max()))


@pytest.mark.parametrize("name,n_prefix", [("c4_bf16", 12345), ("c5_fp8", 20032), ("c5_fp8pv", 20032)])
def test_causal_prefix_invariant_full_size(gpu_lib, name, n_prefix):
    """Causal attention of rows [0, n) depends only on the first n keys: at the
    workload's full size, in the launch configuration the benchmark times, the
    first n rows of the output equal the output of the first n rows alone.  The
    kernels visit the same key tiles in the same order for those rows and keys
    past a row are masked either way, so the two agree bit for bit (FP8: n is a
    multiple of the 64-row scale tile, so the codes and scales agree too)."""
    import torch
    from tiled_attention_13_amd import fwd
    from tiled_attention_13_amd.inputs import WORKLOADS
    w = WORKLOADS[name]
    q, k, v = make_inputs(w)
    tq, tk, tv = (to_device(a, "bf16") for a in (q, k, v))
    o_full, l_full = fwd(tq, tk, tv, causal=True, dtype=w.dtype)
    pq, pk, pv = (t[:, :, :n_prefix].contiguous() for t in (tq, tk, tv))
    o_pre, l_pre = fwd(pq, pk, pv, causal=True, dtype=w.dtype)
    torch.cuda.synchronize()
    assert torch.isfinite(o_full.float()).all() and torch.isfinite(l_full).all()
    assert torch.equal(o_full[:, :, :n_prefix], o_pre), name
    assert torch.equal(l_full[:, :, :n_prefix], l_pre), name


@pytest.mark.parametrize("path", ["bf16", "fp8pv", "bwd", "splitkv", "blocksparse"])
def test_repeated_runs_bit_identical(gpu_lib, path):
    """Every kernel that streams tiles through an LDS ring gives the same bits on
    ten runs of the same input (a race between a tile copy and the reads of the
    stage it overwrites would show up as run-to-run differences)."""
    import torch
    import tiled_attention_13_amd as fa
    from tiled_attention_13_amd.inputs import random_block_mask
    w = Workload("rep", 1, 8, 2048 + 37, 128, "bf16", True, 93)
    q, k, v = make_inputs(w)
    tq, tk, tv = (to_device(a, "bf16") for a in (q, k, v))
    if path == "bwd":
        o, lse = fa.fwd(tq, tk, tv, causal=True)
        tg = to_device(make_grad(w), "bf16")
    if path == "blocksparse":
        nb = (w.N + 63) // 64
        mask = torch.from_numpy(random_block_mask(nb, 0.4, 94)).to("cuda")

    def run():
        if path in ("bf16", "fp8pv"):
            return fa.fwd(tq, tk, tv, causal=True, dtype=path)
        if path == "bwd":
            return fa.bwd(tq, tk, tv, o, tg, lse, causal=True)
        if path == "splitkv":
            return fa.fwd_splitkv(tq, tk, tv, 3, causal=True)
        return fa.fwd_blocksparse(tq, tk, tv, mask, causal=True)

    first = [t.clone() for t in run()]
    for _ in range(9):
        again = run()
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b), path


def test_workspace_allocation_failure_is_reported(gpu_lib, monkeypatch):
    """With FA_TEST_FAIL_ALLOC=1 every entry point that needs a workspace returns
    FA_ERR_OUT_OF_MEMORY (FAError status 9) and writes nothing; the fp32 and bf16
    forwards and the FP8 forward on quantised inputs, which need none, still run
    and write their outputs; afterwards the same calls succeed."""
    import torch
    import tiled_attention_13_amd as fa
    w = Workload("oom", 1, 2, 300, 128, "bf16", True, 95)
    q, k, v = make_inputs(w)
    tq, tk, tv = (to_device(a, "bf16") for a in (q, k, v))
    o, lse = fa.fwd(tq, tk, tv, causal=True)
    tg = to_device(make_grad(w), "bf16")
    mask = torch.ones((5, 5), dtype=torch.uint8, device="cuda")
    calls = {
        "fp8": lambda out: fa.fwd(tq, tk, tv, causal=True, dtype="fp8", out=out),
        "fp8pv": lambda out: fa.fwd(tq, tk, tv, causal=True, dtype="fp8pv", out=out),
        "splitkv": lambda out: fa.fwd_splitkv(tq, tk, tv, 2, causal=True, out=out),
        "blocksparse": lambda out: fa.fwd_blocksparse(tq, tk, tv, mask, causal=True, out=out),
        "bwd": lambda out: fa.bwd(tq, tk, tv, o, tg, lse, causal=True, dq=out),
    }
    monkeypatch.setenv("FA_TEST_FAIL_ALLOC", "1")
    for name, call in calls.items():
        out = torch.full_like(tq, 7.0)
        with pytest.raises(fa.FAError) as e:
            call(out)
        assert e.value.status == 9, name
        torch.cuda.synchronize()
        assert torch.all(out == 7.0), name                    # nothing was enqueued
    q32, k32, v32 = (to_device(a, "f32") for a in (q, k, v))
    fa.fwd(q32, k32, v32, causal=True)                        # no workspace: unaffected
    q8, qs = fa.quant_fp8(tq)
    k8, ks = fa.quant_fp8(tk)
    for name, call in (("bf16", lambda out: fa.fwd(tq, tk, tv, causal=True, out=out)),
                       ("fp8 kernel", lambda out: fa.fwd_fp8(q8, qs, k8, ks, tv, causal=True, out=out))):
        out = torch.full_like(tq, 7.0)
        call(out)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all() and not torch.all(out == 7.0), name
    monkeypatch.delenv("FA_TEST_FAIL_ALLOC")
    for name, call in calls.items():
        call(torch.empty_like(tq))
    torch.cuda.synchronize()
