"""Pins of the oracle's number codecs: E4M3FN decode and bf16 rounding.

The E4M3FN table is checked against its closed form (sign, 4-bit exponent with
bias 7, 3-bit mantissa, subnormals at exponent 0, NaN only at S.1111.111) on
hand-picked codes and against torch's float8_e4m3fn library cast on all 256
codes.  bf16 rounding is checked against torch's float32 -> bfloat16 cast
(round to nearest even) and against hand cases, including ties.
"""

import math

import numpy as np
import pytest
import torch

from oracle import E4M3FN_TABLE, bf16_round, e4m3fn_value


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x38, 1.0), (0x40, 2.0), (0x30, 0.5), (0x48, 4.0),
    (0x7E, 448.0), (0xFE, -448.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9),
    (0x07, 7 * 2.0 ** -9), (0x3C, 1.5), (0x77, 240.0), (0x78, 256.0), (0xB8, -1.0),
])
def test_e4m3fn_closed_form_points(code, value):
    assert e4m3fn_value(code) == value
    assert E4M3FN_TABLE[code] == value


def test_e4m3fn_nan_and_negative_zero():
    assert math.isnan(e4m3fn_value(0x7F)) and math.isnan(e4m3fn_value(0xFF))
    assert e4m3fn_value(0x80) == 0.0 and math.copysign(1.0, e4m3fn_value(0x80)) == -1.0
    assert int(np.isnan(E4M3FN_TABLE).sum()) == 2


def test_e4m3fn_table_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ref == E4M3FN_TABLE) | (np.isnan(ref) & np.isnan(E4M3FN_TABLE))
    assert same.all(), np.nonzero(~same)


def test_e4m3fn_monotone_positive_half():
    pos = E4M3FN_TABLE[:0x7F]
    assert (np.diff(pos) > 0).all()
    assert (E4M3FN_TABLE[0x80:0xFF] == -pos).all()


def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * np.exp(rng.uniform(-40, 40, 20000)),
        rng.standard_normal(2000) * 1e-39,           # float32 subnormals
        np.array([0.0, -0.0, 1.0, 3.0e38, -3.0e38]),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = bf16_round(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_round_ties_to_even_and_overflow():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even significand (1.0)
    assert bf16_round(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even (1 + 2^-6)
    assert bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    # just above the halfway point rounds up
    assert bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    # directly from float64: no double rounding through float32
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30   # float32 would round this to exactly the tie
    assert bf16_round(x) == 1.0 + 2.0 ** -7
    assert bf16_round(3.5e38) == math.inf
    assert bf16_round(-np.inf) == -math.inf
    assert math.isnan(bf16_round(np.nan))
    assert bf16_round(2.0 ** -133) == 2.0 ** -133       # smallest bf16 subnormal
    assert bf16_round(2.0 ** -135) == 0.0               # below half of it
