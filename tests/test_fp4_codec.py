"""Pins of the oracle's FP4 E2M1 codec (CPU only), from the format definition:
the eight magnitudes, every midpoint tie, saturation, NaN, sign, the round
trip of all 16 codes, packing order, and FP4 attention through the oracle
against a dense float64 reference on dequantised values."""

import math

import numpy as np
import pytest
import torch

from oracle import fp4_e2m1 as fp4
from oracle import paged

MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_all_codes_decode_to_the_defined_values():
    for code in range(16):
        expect = MAGNITUDES[code & 7] * (-1.0 if code & 8 else 1.0)
        got = fp4.decode_one(code)
        assert got == expect and math.copysign(1.0, got) == (-1.0 if code & 8 else 1.0)


@pytest.mark.parametrize("x,code", [
    (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),   # ties -> even
    (0.26, 1), (0.74, 1), (2.51, 5), (4.99, 6), (5.01, 7),
    (6.0, 7), (6.5, 7), (1e9, 7), (float("inf"), 7),                            # saturation
    (-1.25, 10), (-0.0, 8), (-1e-30, 8), (-float("inf"), 15),
    (float("nan"), 0),
])
def test_encode_rounding_saturation_and_sign(x, code):
    assert int(fp4.encode(np.array([x]))[0]) == code


def test_round_trip_of_every_code():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(fp4.encode(fp4.decode(codes)), codes)


def test_packing_order():
    codes = np.array([[1, 2, 3, 15]], dtype=np.uint8)
    packed = fp4.pack(codes)
    assert packed.tolist() == [[0x21, 0xF3]]
    assert np.array_equal(fp4.unpack(packed), codes)


def test_division_is_binary32():
    # 1.25 / 0.5 is 2.5 exactly (tie -> 2); 1 / 3 in binary32 then encoded
    assert int(fp4.quantize_f32_div(np.float32(1.25), np.float32(0.5))) == 4
    q = np.divide(np.float32(1.0), np.float32(3.0), dtype=np.float32)
    assert int(fp4.quantize_f32_div(np.float32(1.0), np.float32(3.0))) == int(fp4.encode(q))


def test_fp4_decode_attention_equals_dense_reference():
    rng = np.random.default_rng(21710)
    nb, n_kv, bs, d, n_q = 6, 2, 4, 8, 4
    k = rng.integers(0, 256, size=(nb, n_kv, bs, d // 2), dtype=np.uint8)
    v = rng.integers(0, 256, size=(nb, n_kv, bs, d // 2), dtype=np.uint8)
    ks = np.array([0.7, 1.3], dtype=np.float32)
    vs = np.array([0.25, 2.0], dtype=np.float32)
    qf = rng.standard_normal((1, n_q, d)).astype(np.float32)
    q = torch.from_numpy(qf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    table = np.array([[4, 1, 5]], dtype=np.int32)
    out = paged.decode_attention(q, k, v, table, np.array([10], np.int32), 0.3, paged.FP4, ks, vs)
    # dense: rows of the three blocks, dequantised by hand from the definition
    kd = np.concatenate([k[b] for b in (4, 1, 5)], axis=1)[:, :10]
    vd = np.concatenate([v[b] for b in (4, 1, 5)], axis=1)[:, :10]
    kf = fp4.decode(fp4.unpack(kd)) * ks[:, None, None]
    vf = fp4.decode(fp4.unpack(vd)) * vs[:, None, None]
    qd = torch.from_numpy(qf).to(torch.bfloat16).double().numpy()[0]
    for h in range(n_q):
        g = h // 2
        s = 0.3 * kf[g] @ qd[h]
        w = np.exp(s - s.max())
        w /= w.sum()
        assert np.allclose(out[0, h], w @ vf[g], rtol=1e-12, atol=1e-12)
