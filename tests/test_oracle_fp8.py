"""Pins of the oracle's FP8 E4M3 arithmetic (8-bit KV pool) against the OCP
definition's fixed points, brute force over every code, and torch's own
float8_e4m3fn conversion (a library routine) inside the finite range."""
import numpy as np
import pytest
import torch

from oracle import pa_oracle as O


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x7E, 448.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x3C, 1.5), (0x40, 2.0), (0xB8, -1.0), (0x00, 0.0), (0x77, 240.0),
])
def test_code_values(code, value):
    assert O.e4m3_value(code) == value


def test_nan_codes_and_negative_zero():
    assert np.isnan(O.e4m3_value(0x7F)) and np.isnan(O.e4m3_value(0xFF))
    v = O.e4m3_value(0x80)
    assert v == 0.0 and np.signbit(v)
    assert sum(np.isnan(O.e4m3_value(c)) for c in range(256)) == 2


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),          # halfway 1.0 / 1.125: even mantissa
    (1.1875, 0x3A),          # halfway 1.125 / 1.25: even mantissa
    (2.0 ** -10, 0x00),      # halfway 0 / 2^-9
    (3 * 2.0 ** -10, 0x02),  # halfway 2^-9 / 2^-8
    (448.0, 0x7E), (449.0, 0x7E), (1e9, 0x7E), (-1e9, 0xFE), (464.0, 0x7E),
    (-0.0, 0x80), (1e-30, 0x00),
])
def test_encode_fixed_points(x, code):
    assert int(O.e4m3_encode([x])[0]) == code


def test_encode_nan():
    assert int(O.e4m3_encode([float("nan")])[0]) == 0x7F


def test_every_finite_code_round_trips():
    codes = [c for c in range(256) if not np.isnan(O.e4m3_value(c))]
    vals = np.array([O.e4m3_value(c) for c in codes], dtype=np.float32)
    assert O.e4m3_encode(vals).tolist() == codes


def test_encode_is_nearest_brute_force():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(3000) * 10 ** rng.uniform(-4, 3, 3000),
                        rng.uniform(-500, 500, 1000)]).astype(np.float32)
    got = O.e4m3_values(O.e4m3_encode(x))
    finite = np.array([O.e4m3_value(c) for c in range(256) if not np.isnan(O.e4m3_value(c))])
    for xi, gi in zip(x.astype(np.float64), got):
        target = np.clip(xi, -448.0, 448.0)
        assert abs(gi - target) <= np.min(np.abs(finite - target)) + 0.0


def test_matches_torch_float8_e4m3fn_in_range():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(20000) * 10 ** rng.uniform(-4, 2.6, 20000)).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), ref)


def test_quantize_uses_float32_reciprocal_and_product():
    rng = np.random.default_rng(9)
    x = rng.standard_normal(1000).astype(np.float32)
    scale = 0.0123
    inv = np.float32(1) / np.float32(scale)
    assert np.array_equal(O.quantize_e4m3(x, scale), O.e4m3_encode((x * inv).astype(np.float32)))
    # a value at the pool's largest magnitude maps to 448's code
    assert int(O.quantize_e4m3(np.float32([448 * scale]), scale)[0]) in (0x7E,)


def test_cache_write_and_dequantized_decode():
    """The 8-bit slot write stores the codes of the scaled rows at the slots,
    and the decode over the dequantized pools is the ordinary decode."""
    rng = np.random.default_rng(10)
    nb, hkv, bs, d = 6, 2, 4, 8
    kc = np.zeros((nb, hkv, bs, d), dtype=np.uint8)
    vc = np.zeros_like(kc)
    k_new = rng.standard_normal((3, hkv, d)).astype(np.float32)
    v_new = rng.standard_normal((3, hkv, d)).astype(np.float32)
    O.reshape_and_cache_e4m3(k_new, v_new, [5, -1, 22], kc, vc, 0.02, 0.03)
    assert np.array_equal(kc[1, :, 1], O.quantize_e4m3(k_new[0], 0.02))
    assert np.array_equal(vc[5, :, 2], O.quantize_e4m3(v_new[2], 0.03))
    assert np.count_nonzero(kc) == np.count_nonzero(kc[1, :, 1]) + np.count_nonzero(kc[5, :, 2])
    kd, vd = O.dequantize_e4m3(kc, 0.02), O.dequantize_e4m3(vc, 0.03)
    assert np.allclose(kd[1, :, 1], k_new[0], rtol=0.07, atol=0.02 * 2 ** -9)
