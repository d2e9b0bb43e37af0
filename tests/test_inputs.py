"""Host-side checks: the seeded input recipe and the FLOP/byte calculator."""
import json
import os

import numpy as np
import pytest

from tiled_attention_13_amd.inputs import WORKLOADS, Workload, digest, make_inputs, round_to_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_arithmetic.json")


def test_same_seed_same_tensors_other_seed_differs():
    w = WORKLOADS["c2_bf16"]
    a = make_inputs(w, shape=(1, 2, 64, 32))
    b = make_inputs(w, shape=(1, 2, 64, 32))
    c = make_inputs(w, seed=99, shape=(1, 2, 64, 32))
    assert digest(*a) == digest(*b)
    assert digest(*a) != digest(*c)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(1_000_000).astype(np.float32) * 7,
                        # exact halfway cases between neighbouring bf16 values
                        (np.arange(1, 20001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_to_bf16(x), ref)


def test_recipe_gain_and_spikes():
    w = WORKLOADS["c4_bf16"]
    q, k, v = make_inputs(w, shape=(1, 2, 1000, 16))
    # 1% of the key rows (10 per head) are multiplied by 8
    base = Workload("plain", 1, 2, 1000, 16, "bf16", True, w.seed)
    q0, k0, v0 = make_inputs(base)
    np.testing.assert_array_equal(q, q0)
    np.testing.assert_array_equal(v, v0)
    for h in range(2):
        ratio = np.abs(k[0, h]).sum(axis=1) / np.abs(k0[0, h]).sum(axis=1)
        assert np.sum(np.isclose(ratio, 8.0)) == 10
        assert np.sum(np.isclose(ratio, 1.0)) == 990
    w3 = WORKLOADS["c3_bf16"]
    q3, k3, v3 = make_inputs(w3, shape=(1, 1, 64, 8))
    q1, k1, v1 = make_inputs(Workload("plain", 1, 1, 64, 8, "bf16", True, w3.seed), shape=(1, 1, 64, 8))
    np.testing.assert_array_equal(q3, 2 * q1)
    np.testing.assert_array_equal(k3, 2 * k1)
    np.testing.assert_array_equal(v3, v1)


def test_bf16_workloads_are_representable():
    w = WORKLOADS["c3_bf16"]
    q, k, v = make_inputs(w, shape=(1, 1, 256, 128))
    for a in (q, k, v):
        assert np.all((a.view(np.uint32) & 0xFFFF) == 0)


def test_flop_and_byte_calculator_against_page_arithmetic():
    g = json.load(open(GOLDEN))
    for e in g["entries"]:
        if "d" in e:
            one = Workload("x", 1, 1, e["n"], e["d"], "f32", False, 0).flops()
            got = one / 2 if "one of the two" in e["what"] else one
        else:
            got = e["n"] ** 2 * 4
        assert got == e["value"], e["cite"]
    assert WORKLOADS["c4_bf16"].flops() == 4 * 32 * 16384 ** 2 * 128 / 2
    assert WORKLOADS["c4_bf16"].compulsory_bytes() == 538_968_064
    assert WORKLOADS["c5_fp8"].compulsory_bytes() == 404_815_872
    assert WORKLOADS["c1_f32"].compulsory_bytes() == 263_168


def test_bench_blocksparse_pair_count_matches_oracle():
    import bench
    import oracle
    from tiled_attention_13_amd.inputs import band_global_block_mask, random_block_mask
    for N in (64, 100, 300, 1000):
        nb = (N + 63) // 64
        for m in (band_global_block_mask(nb, 3, 1), random_block_mask(nb, 0.5, N), np.ones((nb, nb), np.uint8)):
            for causal in (False, True):
                assert bench.blocksparse_pairs(m, N, causal) == oracle.visible_pairs(m, N, causal)
