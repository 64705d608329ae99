"""Pins for the oracle's OCP E4M3 codec (CPU only).

The codec is checked against torch's float8_e4m3fn (an independent library
implementation) on every code and on random in-range values, and against
values fixed by the format's definition: the largest finite magnitude 448,
the smallest normal 2**-6, the smallest subnormal 2**-9, signed zero, the
single NaN pattern per sign, ties to even and saturation.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3_decode, e4m3_encode




def torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_on_all_codes():
    ours = e4m3_decode(np.arange(256, dtype=np.uint8))
    ref = torch_decode_all()
    nan_ours = np.isnan(ours)
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ours, nan_ref)
    assert np.flatnonzero(nan_ours).tolist() == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref])
    assert np.array_equal(np.signbit(ours[~nan_ours]), np.signbit(ref[~nan_ref]))


@pytest.mark.parametrize("code,value", [
    (0x7E, 448.0), (0xFE, -448.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9),
    (0x07, 7 * 2.0 ** -9), (0x38, 1.0), (0x39, 1.125), (0x40, 2.0),
    (0x00, 0.0)])
def test_decode_fixed_points(code, value):
    assert e4m3_decode(np.array([code], dtype=np.uint8))[0] == value


def test_negative_zero():
    v = e4m3_decode(np.array([0x80], dtype=np.uint8))[0]
    assert v == 0.0 and math.copysign(1.0, v) < 0
    assert e4m3_encode(np.array([-0.0]))[0] == 0x80


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)],
                     dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    parts = [rng.standard_normal(200000).astype(np.float32) * s
             for s in (1.0, 30.0, 200.0, 2.0 ** -7, 2.0 ** -10)]
    x = np.concatenate(parts)
    x = x[np.abs(x) <= 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = e4m3_encode(x.astype(np.float64))
    # torch keeps the sign of values that round to zero; so do we
    assert np.array_equal(ours, ref)


def test_ties_go_to_even():
    # between 1.0 (m=0) and 1.125 (m=1): 1.0625 -> even m=0
    # between 1.125 and 1.25 (m=2): 1.1875 -> even m=2
    # subnormal grid: 2**-10 is half of the smallest step -> 0 (even)
    #                 3 * 2**-10 is between 1 and 2 steps -> 2 steps
    vals = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10,
                     15.0 * 2.0 ** -10])
    assert e4m3_encode(vals).tolist() == [0x38, 0x3A, 0x00, 0x02, 0x08]
    ref = torch.from_numpy(vals.astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).tolist()
    assert e4m3_encode(vals).tolist() == ref


def test_saturation_and_nan():
    vals = np.array([448.0, 449.0, 464.0, 465.0, 1e6, np.inf, -1e6, -np.inf,
                     np.nan, -np.nan])
    codes = e4m3_encode(vals).tolist()
    assert codes[:8] == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert codes[8] & 0x7F == 0x7F and codes[9] & 0x7F == 0x7F


def test_encode_is_monotone():
    x = np.linspace(-500, 500, 200001)
    dec = e4m3_decode(e4m3_encode(x))
    assert np.all(np.diff(dec) >= 0)
    # nearest: the error never exceeds half the local spacing
    err = np.abs(dec - np.clip(x, -448, 448))
    fin = np.abs(x) <= 448
    spacing = np.where(np.abs(x) < 2.0 ** -6, 2.0 ** -9,
                       2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 1e-30))) - 3))
    assert np.all(err[fin] <= spacing[fin] / 2 + 1e-12)


def test_widening_table_is_the_decoder():
    """to_float64 widens fp8 codes through a table of the decoders' values;
    on every code and on a random array (with NaN codes) it gives the
    decoders' float64 values bit for bit."""
    from oracle.storage import to_float64
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, (37, 64), dtype=np.uint8)
    for kind, dec in (("fp8_e4m3", oracle.e4m3_decode),
                      ("fp8_e5m2", oracle.e5m2_decode)):
        every = np.arange(256, dtype=np.uint8)
        assert to_float64(every, kind).tobytes() == dec(every).tobytes()
        assert to_float64(codes, kind).tobytes() == dec(codes).tobytes()
        assert to_float64(codes, kind).shape == codes.shape
