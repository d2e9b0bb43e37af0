"""Pins of the oracle's e4m3fn codec, per-tile scaling and FP8 attention.

The codec is checked against torch's own ``float8_e4m3fn`` type (all 256
codes decoded; rounding of every representable value, every midpoint and
its neighbours, and a million random values), against values the OCP
format definition fixes (largest finite 448, smallest subnormal 2**-9,
NaN codes), and the scaling against the closed forms of the rule
(scale = 448 / amax; the largest element lands on +-448; error within half
an e4m3 step).
"""
import numpy as np
import pytest

import oracle
from oracle.fp8 import decode_e4m3, encode_e4m3, quantize_tiles

torch = pytest.importorskip("torch")


def _torch_codes(y32):
    t = torch.from_numpy(np.ascontiguousarray(y32, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_decode_fixed_points_of_the_format():
    assert decode_e4m3([0x7E])[0] == 448.0
    assert decode_e4m3([0xFE])[0] == -448.0
    assert decode_e4m3([0x01])[0] == 2.0 ** -9
    assert decode_e4m3([0x07])[0] == 7 * 2.0 ** -9
    assert decode_e4m3([0x08])[0] == 2.0 ** -6
    assert decode_e4m3([0x38])[0] == 1.0
    assert decode_e4m3([0x00])[0] == 0.0 and not np.signbit(decode_e4m3([0x00])[0])
    assert decode_e4m3([0x80])[0] == 0.0 and np.signbit(decode_e4m3([0x80])[0])


def _sweep_values():
    pos = decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2.0                     # exact ties (float32-representable)
    m32 = mids.astype(np.float32)
    around = np.concatenate([np.nextafter(m32, np.float32(0)), m32, np.nextafter(m32, np.float32(1e9))])
    rng = np.random.default_rng(0)
    rnd = np.concatenate([rng.uniform(-448, 448, 500_000),
                          np.exp2(rng.uniform(-12, np.log2(448), 500_000)) * rng.choice([-1, 1], 500_000)])
    vals = np.concatenate([pos, -pos, around, -around, rnd]).astype(np.float32)
    return vals[np.abs(vals) <= 448]


def test_encode_matches_torch_rne():
    y = _sweep_values()
    np.testing.assert_array_equal(encode_e4m3(y), _torch_codes(y))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        encode_e4m3([448.5])
    with pytest.raises(ValueError):
        encode_e4m3([np.nan])


def test_quantize_scale_rule_and_saturation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, 200, 32)).astype(np.float32)
    codes, scale = quantize_tiles(x)
    assert scale.shape == (2, 3, 4) and scale.dtype == np.float32
    for b in range(2):
        for h in range(3):
            for t in range(4):
                tile = x[b, h, 64 * t:64 * (t + 1)]
                amax = float(np.max(np.abs(tile)))
                # division carried out in float64 then rounded once equals the fp32 IEEE quotient
                assert scale[b, h, t] == np.float32(448.0 / amax)
                idx = np.unravel_index(np.argmax(np.abs(tile)), tile.shape)
                c = codes[b, h, 64 * t:64 * (t + 1)][idx]
                assert c == (0xFE if tile[idx] < 0 else 0x7E)
                back = decode_e4m3(codes[b, h, 64 * t:64 * (t + 1)]) / float(scale[b, h, t])
                err = np.abs(back - tile)
                bound = np.maximum(np.abs(tile) * 2.0 ** -4, 2.0 ** -10 / float(scale[b, h, t])) * (1 + 1e-6)
                assert np.all(err <= bound)


def test_partial_tile_uses_only_its_rows():
    x = np.zeros((1, 1, 100, 16), dtype=np.float32)
    x[0, 0, :64] = 10.0
    x[0, 0, 64:] = np.linspace(-0.5, 0.25, 36 * 16, dtype=np.float32).reshape(36, 16)
    codes, scale = quantize_tiles(x)
    assert scale[0, 0, 0] == np.float32(44.8)
    assert scale[0, 0, 1] == np.float32(448.0) / np.float32(0.5)
    assert codes[0, 0, 64, 0] == 0xFE                       # -0.5 is the tile's extreme


def test_zero_tile_is_finite():
    x = np.zeros((1, 1, 64, 8), dtype=np.float32)
    codes, scale = quantize_tiles(x)
    assert scale[0, 0, 0] == np.float32(448.0) / np.float32(1e-6)
    assert np.all(codes == 0)


def test_fp8_attention_equals_attention_on_dequantised_values():
    rng = np.random.default_rng(2)
    shape = (1, 2, 150, 16)
    q = rng.standard_normal(shape).astype(np.float32)
    k = rng.standard_normal(shape).astype(np.float32)
    v = rng.standard_normal(shape)
    q8, qs = quantize_tiles(q)
    k8, ks = quantize_tiles(k)
    qv, kv = decode_e4m3(q8), decode_e4m3(k8)
    q_deq = qv / np.repeat(qs.astype(np.float64), 64, axis=2)[:, :, :150, None]
    k_deq = kv / np.repeat(ks.astype(np.float64), 64, axis=2)[:, :, :150, None]
    for causal in (False, True):
        O, lse = oracle.attention_fp8(qv, qs, kv, ks, v, causal, 0.25)
        O_ref, lse_ref = oracle.attention(q_deq, k_deq, v, causal, 0.25)
        np.testing.assert_allclose(O, O_ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=1e-13)
        # quantisation perturbs the result only slightly relative to the unquantised inputs
        O_raw, _ = oracle.attention(q, k, v, causal, 0.25)
        assert np.max(np.abs(O - O_raw)) < 0.1


# ---------------------------------------------------------------------------
# power-of-two scaled V (FP8 P*V)
# ---------------------------------------------------------------------------

def test_pow2_exponent_definition():
    cases = {448.0: 0, 448.00001: -1, 447.9: 0, 224.0: 1, 224.0001: 0, 1.0: 8, 0.875: 9, 0.8751: 8,
             3.5: 7, 3.50001: 6, 2.0 ** -20: 28, 1e30: -91, 0.0: 0, 1e-39: 127, 2.0 ** -118: 126,
             2.0 ** -119: 127, 1e300: -127}
    for a, e in cases.items():
        assert oracle.pow2_exponent(a) == e, (a, e)
    rng = np.random.default_rng(5)
    a = np.exp(rng.uniform(-40, 40, 100000))      # well inside the clip range
    e = oracle.pow2_exponent(a)
    assert np.all(np.ldexp(a, e) <= 448.0) and np.all(np.ldexp(a, e + 1) > 448.0)


def test_quantize_v_pow2_properties():
    rng = np.random.default_rng(6)
    v = (rng.standard_normal((2, 3, 150, 16)) * np.exp(rng.uniform(-6, 6, (2, 3, 1, 16)))).astype(np.float32)
    v[0, 0, 64:128, 3] = 0.0                                  # an all-zero column of a tile
    codes, exps = oracle.quantize_v_pow2(v)
    assert codes.shape == v.shape and exps.shape == (2, 3, 3, 16)
    assert exps[0, 0, 1, 3] == 0 and np.all(codes[0, 0, 64:128, 3] == 0)
    vals = oracle.dequantize_v_pow2(codes, exps)
    # each value is within half an e4m3 step of V: relative 2^-4 for normals,
    # absolute 2^-10 * 2^-e in the subnormal range
    e_rows = np.repeat(exps, 64, axis=2)[:, :, :150]
    bound = np.maximum(np.abs(v) * 2.0 ** -4, np.ldexp(2.0 ** -10, -e_rows))
    assert np.all(np.abs(vals - v) <= bound * (1 + 1e-12))
    # the largest magnitude of every (tile, column) lands in (224, 448]
    for t in range(3):
        top = np.abs(decode_e4m3(codes[:, :, 64 * t:64 * t + 64])).max(axis=2)
        nz = np.abs(v[:, :, 64 * t:64 * t + 64]).max(axis=2) > 0
        assert np.all(top[nz] > 224 * (1 - 2.0 ** -4)) and np.all(top[nz] <= 448)


def test_quantize_v_pow2_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    v = rng.standard_normal((1, 2, 200, 32)).astype(np.float32) * 3
    codes, exps = oracle.quantize_v_pow2(v)
    e_rows = np.repeat(exps, 64, axis=2)[:, :, :200]
    scaled = np.ldexp(v.astype(np.float64), e_rows).astype(np.float32)   # exact: powers of two
    ref = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)
