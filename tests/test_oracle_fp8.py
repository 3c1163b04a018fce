"""Pins of the oracle's FP8 E4M3 arithmetic (8-bit KV pool) against the OCP
definition's fixed points, brute force over every code, torch's own
float8_e4m3fn conversion (a library routine) inside the finite range, and
exact rational arithmetic for the quantization rule (nearest code to the
exact quotient x / scale)."""
from fractions import Fraction

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


def _torch_code_values():
    """Values of the 127 non-negative finite codes from torch's own
    float8_e4m3fn type (a library routine, independent of the oracle)."""
    vals = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    return [Fraction(float(v)) for v in vals]


def _exact_code(x: float, s: float, values) -> int:
    """Nearest code to the exact rational x / s (ties to the even code),
    saturating at 448, by exact comparison with every code value."""
    q = Fraction(x) / Fraction(s)
    a = min(abs(q), values[-1])
    best = min(range(0x7F), key=lambda c: (abs(values[c] - a), c % 2))
    return best | (0x80 if q < 0 or (q == 0 and np.signbit(x)) else 0)


def _near_midpoint_inputs(scales, rng):
    """float32 values x within a few ulps of m * s for every midpoint m
    between adjacent codes and every scale s (so x / s sits on or right
    beside a rounding boundary), both signs."""
    values = [float(v) for v in _torch_code_values()]
    xs, ss = [], []
    for s in scales:
        s32 = np.float32(s)
        for k in range(0x7E):
            m = (values[k] + values[k + 1]) / 2
            c = np.float32(m * float(s32))
            for step in (-2, -1, 0, 1, 2):
                x = c
                for _ in range(abs(step)):
                    x = np.nextafter(x, np.float32(np.inf if step > 0 else -np.inf))
                sign = np.float32(-1 if rng.random() < 0.5 else 1)
                xs.append(np.float32(x * sign))
                ss.append(s32)
    return np.array(xs, dtype=np.float32), np.array(ss, dtype=np.float32)


SCALES = [0.37, 0.11, 0.0123, 1 / 3, 0.005, 1.0, 3.0, 7e-3, 0.125, 2.0 ** -20, 1234.5]


def test_quantize_is_nearest_code_of_exact_quotient():
    """quantize_e4m3 against exact rational arithmetic: for inputs on or
    beside every rounding boundary of 11 scales, the code is the nearest one
    to the exact x / scale (ties to the even code)."""
    rng = np.random.default_rng(9)
    values = _torch_code_values()
    xs, ss = _near_midpoint_inputs(SCALES, rng)
    got = np.concatenate([O.quantize_e4m3(xs[ss == s], float(s)) for s in np.unique(ss)])
    xs_o = np.concatenate([xs[ss == s] for s in np.unique(ss)])
    ss_o = np.concatenate([ss[ss == s] for s in np.unique(ss)])
    want = [_exact_code(float(x), float(s), values) for x, s in zip(xs_o, ss_o)]
    assert got.tolist() == want
    # exact ties (power-of-two scales make m * s a float32): ties go to the
    # even code
    ties = [(np.float32(m * 0.125), 0.125) for m in (1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10)]
    for x, s in ties:
        assert int(O.quantize_e4m3(np.array([x]), s)[0]) == _exact_code(float(x), s, values)
    assert [int(O.quantize_e4m3(np.array([x]), s)[0]) for x, s in ties] == [0x38, 0x3A, 0x00, 0x02]


def test_quantize_rule_is_the_quotient_not_the_reciprocal_product():
    """Inputs where x / s and x * float32(1 / s) (rounded to float32) round to
    different codes: the oracle gives the quotient's code, so the test says
    which rule is in force."""
    rng = np.random.default_rng(10)
    values = _torch_code_values()
    xs, ss = _near_midpoint_inputs(SCALES, rng)
    recip = np.array([O.e4m3_encode([np.float32(x * (np.float32(1) / s))])[0]
                      for x, s in zip(xs, ss)])
    exact = np.array([_exact_code(float(x), float(s), values) for x, s in zip(xs, ss)])
    differ = recip != exact
    assert differ.sum() >= 20
    got = np.array([O.quantize_e4m3(np.array([x]), float(s))[0] for x, s in zip(xs[differ], ss[differ])])
    assert np.array_equal(got, exact[differ])
    # a value at the pool's largest magnitude maps to 448's code
    assert int(O.quantize_e4m3(np.float32([448 * 0.0123]), 0.0123)[0]) == 0x7E


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
