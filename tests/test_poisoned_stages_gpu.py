"""Race check of the LDS rings: the library built with FA_POISON_STAGES=1
(libfa_poisoned.so) fills every 1 KiB LDS block with NaN right before a copy
into it is issued, i.e. just after the barrier that ends the last read of
the stage's previous tile.  A read that lagged behind that barrier or ran
ahead of the copy's wait would see NaN; with no such race both builds give the
same bits.  Covered: the bf16 d=128 forward (128-key slots, separate K and V
rings), the FP8 d=128 forward (three K stages, copies issued by the
matrix-core group, K two tiles ahead), the bf16 d=32 forward (256-key stages,
two-stage ring, wrapped twice at N = 1037), the 64-key LDS-DMA kernels (bf16 at
d = 64, FP8 at d = 32 and 64, FP8 P*V, split-KV partials) and the backward's
rings (at d = 128 the dK/dV kernel's three-stage ring of rows read both ways,
and the dQ kernel's rings), at d = 32, 64 and 128 and small ragged shapes
spanning several tiles."""
import os

import pytest

from parity_util import to_device
from tiled_attention_13_amd.inputs import Workload, make_grad, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def poisoned():
    from tiled_attention_13_amd import _binding
    from tiled_attention_13_amd.build import LIB_POISONED
    if not os.path.exists(LIB_POISONED):
        pytest.fail("libfa_poisoned.so is not built (run `python -m tiled_attention_13_amd.build`)")
    return _binding.load_library(LIB_POISONED)


def _with_lib(lib, fn):
    from tiled_attention_13_amd import _binding
    saved = _binding.load()
    _binding._lib = lib
    try:
        return fn()
    finally:
        _binding._lib = saved


@pytest.mark.parametrize("path", ["bf16", "fp8", "fp8pv", "splitkv", "bwd"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_poisoned_build_gives_the_same_bits(gpu_lib, poisoned, path, causal, d):
    import torch
    import tiled_attention_13_amd as fa
    w = Workload("poison", 1, 3, 1000 + 37, d, "bf16", causal, 97)
    q, k, v = make_inputs(w)
    tq, tk, tv = (to_device(a, "bf16") for a in (q, k, v))
    if path == "bwd":
        o, lse = fa.fwd(tq, tk, tv, causal=causal)
        tg = to_device(make_grad(w), "bf16")

    def run():
        if path in ("bf16", "fp8", "fp8pv"):
            r = fa.fwd(tq, tk, tv, causal=causal, dtype=path)
        elif path == "splitkv":
            r = fa.fwd_splitkv(tq, tk, tv, 3, causal=causal)
        else:
            r = fa.bwd(tq, tk, tv, o, tg, lse, causal=causal)
        torch.cuda.synchronize()
        return [t.clone() for t in r]

    normal = run()
    checked = _with_lib(poisoned, run)
    for a, b in zip(normal, checked):
        assert torch.isfinite(a.float()).all(), path
        assert torch.equal(a, b), path
