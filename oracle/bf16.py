"""bfloat16 bit patterns <-> float64, exact (TEST INFRASTRUCTURE, oracle).

The pages store BF16 keys and values ([SMTS] section "Quantifying the KV-Cache
Memory Wall": p = 2 bytes for BF16). bfloat16 is the upper half of an IEEE
binary32 pattern, so widening is a 16-bit left shift of the pattern followed by
an exact float32 -> float64 conversion.

Pins: tests/test_oracle_pins.py compares `to_f64` with torch's own bfloat16
-> float64 conversion for all 65,536 patterns (a library routine), and checks
named values (0x3F80 = 1.0, 0xC000 = -2.0, 0x0001 = 2**-133, 0x7F80 = +inf).
"""

import numpy as np


def to_f64(bits):
    """Widen bfloat16 bit patterns (uint16 array) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    wide = b.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return wide.view(np.float32).astype(np.float64)


def to_f32(bits):
    """Widen bfloat16 bit patterns (uint16 array) to float32 exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def nan_bits():
    """The quiet-NaN bfloat16 pattern used to poison unused cache memory."""
    return np.uint16(0x7FC0)
