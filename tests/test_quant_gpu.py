"""GPU FP8 quantisation is bit-exact with the oracle's (codes and scales), and
the two FP8 entry points agree with each other."""
import numpy as np
import pytest

from oracle.fp8 import quantize_tiles
from parity_util import compare, oracle_forward, to_device
from tiled_attention_13_amd.inputs import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def _gpu_quant(x):
    import torch
    from tiled_attention_13_amd import quant_fp8
    codes, scale = quant_fp8(to_device(x, "bf16"))
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scale.cpu().numpy()


@pytest.mark.parametrize("N,d", [(1, 32), (63, 64), (64, 128), (100, 128), (1000, 32), (4097, 64)])
def test_quant_bit_exact_small(gpu_lib, N, d):
    w = Workload("q", 2, 3, N, d, "fp8", False, 11 + N)
    q, k, _ = make_inputs(w)
    x = np.concatenate([q, 37.0 * k], axis=0)        # mixed magnitudes
    x[0, 0, :min(N, 64)] = 0.0                        # an all-zero tile
    x[1, 1, 0, 0] = -x[1, 1, 0, 0] - 1e3              # a tile dominated by one value
    x = x.astype(np.float32)
    from tiled_attention_13_amd.inputs import round_to_bf16
    x = round_to_bf16(x)
    codes, scale = _gpu_quant(x)
    codes_ref, scale_ref = quantize_tiles(x)
    np.testing.assert_array_equal(scale, scale_ref)
    np.testing.assert_array_equal(codes, codes_ref)


def test_quant_bit_exact_full_workload(gpu_lib):
    w = WORKLOADS["c5_fp8"]
    q, k, _ = make_inputs(w)
    for x in (q, k):
        codes, scale = _gpu_quant(x)
        codes_ref, scale_ref = quantize_tiles(x)
        np.testing.assert_array_equal(scale, scale_ref)
        np.testing.assert_array_equal(codes, codes_ref)


def test_fp8_entry_points_agree(gpu_lib):
    import torch
    from tiled_attention_13_amd import fwd, fwd_fp8, quant_fp8
    w = Workload("e", 2, 2, 777, 128, "fp8", True, 21)
    q, k, v = make_inputs(w)
    tq, tk, tv = (to_device(a, "bf16") for a in (q, k, v))
    o1, l1 = fwd(tq, tk, tv, causal=True, dtype="fp8")
    q8, qs = quant_fp8(tq)
    k8, ks = quant_fp8(tk)
    o2, l2 = fwd_fp8(q8, qs, k8, ks, tv, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, lse_ref = oracle_forward(q, k, v, "fp8", True, w.softmax_scale)
    compare(o2.float().cpu().numpy().astype(np.float64), l2.cpu().numpy().astype(np.float64),
            o_ref, lse_ref, "fp8", "fwd_fp8")
