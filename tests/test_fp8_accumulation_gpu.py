"""How the e4m3 matrix cores sum their products, seen through fa_fwd_fp8.

With one query and one key (N = 1) and unit tile scales the softmax has a
single term, so lse_0 = S_00 = softmax_scale * (q8 . k8) exactly and O_0 =
V_0: the score is the only thing under test.  The codes are chosen so that
the exact dot product needs more than 14 significant bits: one product of
2^10 (16 x 64) and seven products of 2^-6 (0.125 x 0.125).

* With the small products at head dims 8..15 and the large one at dim 0, the
  lse is exact up to fp32 rounding.
* With all eight at dims 0..7, the small products vanish: the e4m3 MFMA adds
  each run of 8 consecutive products of a lane's operand aligned to the
  largest of them, keeping about 14 bits (a product 2^-3 below a 2^10 one
  survives, 2^-5 does not), before it accumulates in fp32.

The fp32 scale, exp2 and log2 steps are exact or nearly so here, so the
error of the second case is the matrix core's.  This is why the FP8 lse
tolerance grows with the size of the logits (lse within 1e-3 plus 2^-13 of
the largest |lse|): at the FP8 workload's logits (|S| below about 10) that is
still 1e-3, at logits near 70 it is not.  The FP8 page of the sources keeps
"the core computation in FP32" (Triton walkthrough page, section 4.1); on
this hardware the per-product sums inside an MFMA are narrower than that.
"""
import numpy as np
import pytest

from oracle.fp8 import decode_e4m3

pytestmark = pytest.mark.gpu

_CODES = np.arange(256, dtype=np.uint8)
_VALUES = decode_e4m3(_CODES)


def _code(x: float) -> int:
    hit = np.nonzero(_VALUES == x)[0]
    assert hit.size, x
    return int(hit[0])


def _run(d, q8, k8, scale, causal):
    import torch
    import tiled_attention_13_amd as fa
    tq = torch.from_numpy(q8.reshape(1, 1, 1, d)).cuda()
    tk = torch.from_numpy(k8.reshape(1, 1, 1, d)).cuda()
    g = torch.Generator().manual_seed(17)
    v = torch.randn((1, 1, 1, d), generator=g).to(torch.bfloat16).cuda()
    one = torch.ones((1, 1, 1), dtype=torch.float32, device="cuda")
    o, lse = fa.fwd_fp8(tq, one, tk, one, v, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, v)                 # one key: O_0 = V_0
    return float(lse.item())


def _codes(d, small_dims):
    q8 = np.zeros(d, np.uint8)
    k8 = np.zeros(d, np.uint8)
    q8[0], k8[0] = _code(16.0), _code(64.0)          # 2^10
    for j in small_dims:
        q8[j], k8[j] = _code(0.125), _code(0.125)    # 2^-6 each
    exact = float(np.dot(decode_e4m3(q8), decode_e4m3(k8)))
    return q8, k8, exact


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [1.0, 1.0 / 64])
def test_products_in_other_groups_of_eight_are_exact(gpu_lib, d, causal, scale):
    q8, k8, exact = _codes(d, range(8, 15))
    assert exact == 1024.0 + 7 * 2.0 ** -6
    lse = _run(d, q8, k8, scale, causal)
    # fp32: scale * log2(e) product, exp2 of the residual, log2, times ln 2
    assert abs(lse - scale * exact) <= 8 * 2.0 ** -24 * scale * exact + 1e-6, (lse, scale * exact)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [1.0, 1.0 / 64])
def test_small_products_within_a_group_of_eight_are_dropped(gpu_lib, d, causal, scale):
    q8, k8, exact = _codes(d, range(1, 8))
    lse = _run(d, q8, k8, scale, causal)
    truncated = 1024.0                                  # the seven 2^-6 products lost
    assert abs(lse - scale * truncated) <= 8 * 2.0 ** -24 * scale * exact + 1e-6, (lse, scale * truncated)
    # the dropped part is 7 * 2^-6 / 1024 < 2^-13 of the score, inside the FP8 lse bound
    assert abs(lse - scale * exact) <= 1e-3 + 2.0 ** -13 * scale * exact
    if scale == 1.0 / 64:
        assert abs(lse - scale * exact) > 1e-3           # ... but outside a flat 1e-3 at lse = 16


@pytest.mark.parametrize("d", [64, 128])
def test_fourteen_bits_survive(gpu_lib, d):
    """A single product 2^-3 below a 2^10 one in the same group is kept exactly."""
    q8 = np.zeros(d, np.uint8)
    k8 = np.zeros(d, np.uint8)
    q8[0], k8[0] = _code(16.0), _code(64.0)
    q8[3], k8[3] = _code(0.5), _code(0.25)               # 2^-3
    exact = float(np.dot(decode_e4m3(q8), decode_e4m3(k8)))
    lse = _run(d, q8, k8, 1.0, False)
    assert abs(lse - exact) <= 8 * 2.0 ** -24 * exact, (lse, exact)
