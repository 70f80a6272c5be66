"""OCP FP8 E4M3FN codec, written from the format definition (TEST INFRASTRUCTURE, oracle).

The pages store FP8 E4M3 keys and values with per-head scaling factors
([SMTS] section "Technical Q&A", question on FP8 KV-cache quantization;
[LLMI] section "5. Mathematics: Sizing the KV Cache", p = 1 for FP8). They
name neither the E4M3 variant nor the rounding. Readings adopted here:

  * variant: OCP E4M3FN -- 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent field 0 encodes subnormals m/8 * 2**-6; the pattern
    S.1111.111 is NaN; there are no infinities; the largest finite magnitude
    is 1.75 * 2**8 = 448.
  * encode: round to nearest, ties to the code with an even last mantissa
    bit; every finite or infinite magnitude above 448 saturates to +-448;
    NaN encodes as 0x7F. The sign of the input is kept (so -0.0 -> 0x80).

Pins (tests/test_fp8_codec.py): named codes (0x7E = 448, 0x08 = 2**-6,
0x01 = 2**-9, 0x38 = 1.0, 0x7F = NaN, 0x80 = -0.0); all 256 decodes against
torch's float8_e4m3fn -> float64 conversion (a library routine); the encoder
against torch's round-to-nearest-even cast for every bfloat16 pattern whose
magnitude is at most 448, times several scales; saturation above 448; the
identity round trip of every finite code; hand-picked ties.
"""

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = np.uint8(0x7F)


def decode_one(code):
    """Value of one E4M3FN code as a Python float (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * (mant / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


# Table of all 256 decoded values, built one code at a time from the definition.
DECODE_TABLE = np.array([decode_one(c) for c in range(256)], dtype=np.float64)

# Non-negative finite magnitudes in code order 0x00..0x7E; they are strictly
# increasing with the code, which the encoder relies on.
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = DECODE_TABLE[:0x7F]


def decode(codes):
    """Decode an array of E4M3FN codes (uint8) to float64."""
    c = np.asarray(codes, dtype=np.uint8)
    return DECODE_TABLE[c]


def encode(x):
    """Encode float values (given as float32 or float64) to E4M3FN codes.

    Round to nearest representable magnitude, ties to even code; saturate
    magnitudes above 448 (including infinity) to 448; NaN -> 0x7F.
    """
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    nan = np.isnan(flat)
    neg = np.signbit(flat)
    mag = np.abs(flat)
    mag = np.where(nan, 0.0, mag)
    sat = mag >= MAX_FINITE
    # index of the largest representable magnitude <= mag
    lo = np.searchsorted(_POS_VALUES, mag, side="right") - 1
    lo = np.clip(lo, 0, 0x7E)
    hi = np.clip(lo + 1, 0, 0x7E)
    lo_v = _POS_VALUES[lo]
    hi_v = _POS_VALUES[hi]
    d_lo = mag - lo_v
    d_hi = hi_v - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (lo % 2 == 1))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(sat, np.uint8(0x7E), code)
    code = np.where(neg, code | np.uint8(0x80), code)
    code = np.where(nan, NAN_CODE, code)
    out[:] = code
    return out.reshape(x.shape)


def quantize_f32_div(x_f32, scale_f32):
    """code = encode(float32(x / s)) with IEEE float32 division.

    This is the FP8 store of one key or value element under a per-head scale
    s: the element is divided by its head's scale in binary32 (correctly
    rounded) and the quotient is encoded.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    s = np.asarray(scale_f32, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = np.divide(x, s, dtype=np.float32)
    return encode(q)
