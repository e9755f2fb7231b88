"""Oracle: FP8 E4M3 KV-cache codec (test infrastructure).

Page "TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x Faster on Jetson AGX Thor",
section "Using NVFP4 quantization to accelerate Qwen3.6-27B inference": the submitted model keeps
its KV cache in FP8 (while weights and activations are NVFP4), so that long agent contexts take
less of the device's memory.  The pages name no FP8 variant, scale or rounding; the reading taken
here is the plainest one, in the same style as the NVFP4 quantizer of this package:

* format: E4M3FN (the FP8 variant with 448 as its largest finite value);
* one static, calibrated fp32 decode scale s per KV tensor, supplied by the caller (a calibration
  sets s = fl32(amax / 448) so the largest cached value lands on the largest code);
* encode, per element in correctly rounded float32:  inv = (s == 0) ? 0 : fl32(1 / s),
  y = fl32(x * inv),  q = E4M3(y) rounded to nearest even, saturating at +-448, with the sign
  bit of y (so -0 encodes to 0x80);
* decode: x_hat = fl32(e4m3(q) * s) as float32, optionally rounded to bfloat16 (nearest even).

Pinned by tests/test_oracle_kvfp8.py: hand-worked elements (tests/golden/kv_fp8_cases.txt), exact
round trips of every representable value under power-of-two scales, torch's float8_e4m3fn and
bfloat16 casts (library routines) inside the range where they agree with the definition, and the
half-step error bound.  Parity unpinned by the pages: the FP8 variant and the scale are readings.
"""
from __future__ import annotations

import numpy as np

from . import formats as F

E4M3_MAX = F.E4M3_MAX


def calibrated_scale(x) -> np.float32:
    """Static decode scale from calibration data: fl32(amax / 448) (0 for all-zero data)."""
    x = np.asarray(x, dtype=np.float32)
    return np.float32(np.float32(np.max(np.abs(x))) / np.float32(E4M3_MAX)) if x.size else np.float32(0)


def encode(x, s) -> np.ndarray:
    """float32 (or bf16-valued) x -> E4M3FN bytes with decode scale s."""
    x = np.asarray(x, dtype=np.float32)
    s = np.float32(s)
    inv = np.float32(0) if s == 0 else np.float32(np.float32(1) / s)
    with np.errstate(over="ignore"):
        y = (x * inv).astype(np.float32)       # one correctly rounded float32 product
    return F.encode_e4m3(y)


def decode_f32(q, s) -> np.ndarray:
    """E4M3FN bytes -> float32 fl32(e4m3(q) * s)."""
    v = F.decode_e4m3(q).astype(np.float32)   # exact: every E4M3 value is a float32
    return (v * np.float32(s)).astype(np.float32)


def f32_to_bf16_bits(v) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (finite inputs)."""
    b = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def decode_bf16_bits(q, s) -> np.ndarray:
    """E4M3FN bytes -> bfloat16 bit patterns of fl32(e4m3(q) * s), rounded to nearest even."""
    return f32_to_bf16_bits(decode_f32(q, s))
