"""FP4 E2M1 codec, written from the format definition (TEST INFRASTRUCTURE, oracle).

The pages price a 4-bit KV cache at half a byte per element ([MTKV] "The
Anatomy of the KV-Cache Memory Wall": P_bytes = 0.5 for FP4) and list INT4
KV quantization among the engines ([LLMI] "8. Design Alternatives"); they fix
neither the format nor the scaling. Readings adopted here:

  * format: E2M1 -- 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit;
    exponent field 0 encodes the subnormal m/2; there are no infinities and no
    NaN; the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6;
  * scaling: one float32 scale per (K or V, KV head), as for FP8, so the
    cache holds exactly half a byte per element;
  * encode: round to nearest, ties to the code with an even mantissa bit;
    magnitudes above 6 (infinity included) saturate to 6; NaN stores +0
    (the format has no NaN); the sign is kept (-0.0 -> 0x8);
  * packing: element 2i of a row is the low nibble of byte i, element 2i+1
    the high nibble.

Pins (tests/test_fp4_codec.py): the eight magnitudes from the definition
and their negatives; all 16 decodes against the magnitudes listed above;
hand-picked ties at every midpoint; saturation; the identity round trip of
every code; packing order.
"""

import numpy as np

MAX_FINITE = 6.0


def decode_one(code):
    """Value of one E2M1 code (0..15) as a Python float."""
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    exp_field = (code >> 1) & 0x3
    mant = code & 0x1
    if exp_field == 0:
        return sign * mant * 0.5
    return sign * (1.0 + mant / 2.0) * 2.0 ** (exp_field - 1)


DECODE_TABLE = np.array([decode_one(c) for c in range(16)], dtype=np.float64)
_POS_VALUES = DECODE_TABLE[:8]          # strictly increasing with the code


def decode(codes):
    """Decode an array of E2M1 codes (0..15) to float64."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def encode(x):
    """Encode float values to E2M1 codes (uint8 holding 0..15)."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    nan = np.isnan(flat)
    neg = np.signbit(flat) & ~nan
    mag = np.where(nan, 0.0, np.abs(flat))
    lo = np.clip(np.searchsorted(_POS_VALUES, mag, side="right") - 1, 0, 7)
    hi = np.clip(lo + 1, 0, 7)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (lo % 2 == 1))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(mag >= MAX_FINITE, np.uint8(7), code)
    code = np.where(neg, code | np.uint8(0x8), code)
    return code.reshape(x.shape)


def quantize_f32_div(x_f32, scale_f32):
    """code = encode(float32(x / s)), the division in IEEE binary32."""
    x = np.asarray(x_f32, dtype=np.float32)
    s = np.asarray(scale_f32, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = np.divide(x, s, dtype=np.float32)
    return encode(q)


def pack(codes):
    """[..., 2n] codes -> [..., n] bytes (element 2i in the low nibble)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack(packed):
    """[..., n] bytes -> [..., 2n] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
