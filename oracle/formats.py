"""Oracle: decode and encode the two NVFP4 element formats (test infrastructure).

E2M1 (the 4-bit element code) and E4M3FN (the 8-bit block scale), written from
their public bit definitions.  NVFP4 is the 4-bit floating-point format the
page "TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x
Faster on Jetson AGX Thor" uses for weights and activations (section "Using
NVFP4 quantization to accelerate Qwen3.6-27B inference"); the pages do not
spell out its bits, so the definition used here is the public one:

* E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.  The eight
  magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* E4M3FN: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
  exponent 0 is subnormal (m/8 * 2^-6); no infinities; 0x7F/0xFF are NaN;
  the largest finite magnitude is 448 (0x7E).

Encoders are nearest-value searches over the decoded tables.  A value exactly
half way between two neighbours goes to the code whose lowest bit is 0
(round-to-nearest-even).  Magnitudes past the largest finite value saturate to
it (6 for E2M1, 448 for E4M3).  The sign bit is the input's sign bit, so -0.0
encodes to a negative-zero code.  NaN inputs are outside the contract and raise.
"""
from __future__ import annotations

import numpy as np

# The eight E2M1 magnitudes, indexed by the three low code bits.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0


def decode_e2m1(codes) -> np.ndarray:
    """4-bit codes (any integer array, values 0..15) -> float64 values."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 15)):
        raise ValueError("E2M1 codes must be in 0..15")
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where(c & 8, -mag, mag)


def decode_e4m3(b) -> np.ndarray:
    """E4M3FN bytes -> float64 values (NaN for 0x7F / 0xFF)."""
    b = np.asarray(b).astype(np.int64)
    if np.any((b < 0) | (b > 255)):
        raise ValueError("E4M3 bytes must be in 0..255")
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))
    subnormal = np.ldexp(m / 8.0, -6)
    v = np.where(e == 0, subnormal, normal)
    v = np.where((b & 0x7F) == 0x7F, np.nan, v)
    return np.where(b & 0x80, -v, v)


# Non-negative finite E4M3 values in code order 0x00..0x7E; the order is also
# ascending in value, which the nearest search below relies on.
_E4M3_POS = decode_e4m3(np.arange(0x7F))
assert np.all(np.diff(_E4M3_POS) > 0)
_E2M1_POS = E2M1_MAGNITUDES  # codes 0..7, ascending


def _nearest_even(mag: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the nearest entry of the ascending `table` to each magnitude.

    Ties go to the even index; magnitudes beyond the last entry take the last.
    Distances are taken in float64; near a decision boundary the float32 input
    and the table entry are close in exponent, so the differences are exact.
    """
    hi = np.clip(np.searchsorted(table, mag, side="left"), 1, len(table) - 1)
    lo = hi - 1
    d_lo = mag - table[lo]
    d_hi = table[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    return np.where(mag >= table[-1], len(table) - 1, idx)


def encode_e2m1(y) -> np.ndarray:
    """float values -> E2M1 codes (uint8 in 0..15), RNE with saturation at +-6."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.isnan(y)):
        raise ValueError("NaN is outside the NVFP4 contract")
    idx = _nearest_even(np.abs(y), _E2M1_POS)
    return (idx | np.where(np.signbit(y), 8, 0)).astype(np.uint8)


def encode_e4m3(v) -> np.ndarray:
    """float values -> E4M3FN bytes (uint8), RNE with saturation at +-448 (never NaN)."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)):
        raise ValueError("NaN is outside the NVFP4 contract")
    idx = _nearest_even(np.abs(v), _E4M3_POS)
    return (idx | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)
