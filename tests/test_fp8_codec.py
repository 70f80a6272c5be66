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
    # The quotient is rounded to binary32 before it is encoded. Here the float32
    # quotient is exactly 19/1024, the midpoint of codes 0x09 (9/512) and 0x0A
    # (10/512), which ties to the even code 0x0A; the float64 quotient lies just
    # below the midpoint and would give 0x09.
    x = np.float32(0.019002437591552734)
    s = np.float32(1.024131417274475)
    q32 = np.divide(x, s, dtype=np.float32)
    assert q32 == np.float32(19 / 1024)
    assert float(x) / float(s) < 19 / 1024
    assert fp8.quantize_f32_div(np.array([x]), s)[0] == 0x0A
    tq = torch.tensor([x]) / torch.tensor([s])            # torch's binary32 division and cast
    assert tq.to(torch.float8_e4m3fn).view(torch.uint8).item() == 0x0A


def test_fp8_decode_attention_equals_dense_reference():
    # paged FP8 attention against a dense float64 computation whose values are
    # decoded by torch's float8_e4m3fn conversion and scaled per KV head
    from oracle import paged
    rng = np.random.default_rng(21711)
    nb, n_kv, bs, d, n_q = 6, 2, 4, 8, 4
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    k = rng.choice(finite, size=(nb, n_kv, bs, d)).astype(np.uint8)
    v = rng.choice(finite, size=(nb, n_kv, bs, d)).astype(np.uint8)
    ks = np.array([0.007, 0.011], dtype=np.float32)
    vs = np.array([0.25, 2.0], dtype=np.float32)
    qf = rng.standard_normal((1, n_q, d)).astype(np.float32)
    q = torch.from_numpy(qf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    table = np.array([[4, 1, 5]], dtype=np.int32)
    out = paged.decode_attention(q, k, v, table, np.array([10], np.int32), 0.3, paged.FP8, ks, vs)

    def torch_decode(codes):
        return torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()

    kd = np.concatenate([k[b] for b in (4, 1, 5)], axis=1)[:, :10]
    vd = np.concatenate([v[b] for b in (4, 1, 5)], axis=1)[:, :10]
    kf = torch_decode(kd) * ks.astype(np.float64)[:, None, None]
    vf = torch_decode(vd) * vs.astype(np.float64)[:, None, None]
    qd = torch.from_numpy(qf).to(torch.bfloat16).double().numpy()[0]
    for h in range(n_q):
        g = h // 2
        sc = 0.3 * kf[g] @ qd[h]
        w = np.exp(sc - sc.max())
        w /= w.sum()
        assert np.allclose(out[0, h], w @ vf[g], rtol=1e-12, atol=1e-12)
