"""Pins of the oracle's FP8 E4M3FN codec (CPU only).

Expected values come from the format definition written out by hand
(tests/golden/fp8_e4m3fn_named.json), from torch's float8_e4m3fn conversion
(a library routine: exact decode, round-to-nearest-even encode that does not
saturate), and from exhaustive properties (round trip of every finite code).
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import fp8_e4m3 as fp8
from oracle import bf16


def _golden(golden_dir):
    return json.load(open(os.path.join(golden_dir, "fp8_e4m3fn_named.json")))


def test_named_codes(golden_dir):
    g = _golden(golden_dir)
    for code, val in g["codes"].items():
        got = fp8.decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        assert got == val and np.signbit(got) == np.signbit(val), code
    for code in g["nan_codes"]:
        assert np.isnan(fp8.decode(np.array([int(code, 16)], dtype=np.uint8))[0])


def test_all_256_decodes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp8.decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.encode(fp8.decode(codes)), codes)


def test_ties_and_saturation(golden_dir):
    g = _golden(golden_dir)
    for x, code in list(g["ties"].items()) + list(g["saturating"].items()):
        assert fp8.encode(np.array([float(x)]))[0] == int(code, 16), x
    assert fp8.encode(np.array([np.nan]))[0] == 0x7F


@pytest.mark.parametrize("scale", [1.0, 0.5, 3.0, 4.2 / 448, 5.1 / 448, 0.0071])
def test_encoder_matches_torch_on_every_bf16_pattern(scale):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16.to_f32(pats)
    finite = np.isfinite(x)
    ours = fp8.quantize_f32_div(x[finite], np.float32(scale))
    with np.errstate(over="ignore"):
        q = (x[finite] / np.float32(scale)).astype(np.float32)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    inside = np.abs(q) < 464.0      # torch rounds (448, 464) to 448 by RNE and returns NaN at and above 464
    assert np.array_equal(ours[inside], ref[inside])
    over = ~inside
    assert np.all((ours[over] & 0x7F) == 0x7E)
    assert np.array_equal(ours[over] >> 7, np.signbit(q[over]).astype(np.uint8))


def test_encoder_division_is_binary32():
    # x / s is rounded to float32 before encoding: a quotient that is a tie only in
    # float64 must follow the float32 result.
    x = np.float32(1.0000001)
    s = np.float32(0.94117647)
    q32 = np.float32(x / s)
    assert fp8.quantize_f32_div(np.array([x]), s)[0] == fp8.encode(np.array([q32]))[0]
