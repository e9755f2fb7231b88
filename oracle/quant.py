"""Oracle: NVFP4 quantization, packing and dequantization (test infrastructure).

The steps follow the NVFP4 definition (E2M1 codes, an E4M3 scale per 16
contiguous K-elements, one fp32 per-tensor scale) applied to both weights and
activations, as the page "TensorRT Edge-LLM Completes the MLPerf Edge Agentic
Benchmark 6.4x Faster on Jetson AGX Thor", section "Using NVFP4 quantization to
accelerate Qwen3.6-27B inference", describes (weights quantized once after
training; activations also NVFP4).  The pages give no formulas; the readings
below are the plainest ones consistent with the format:

* per-tensor (global) decode scale g = fl32(amax|x| / 2688), 2688 = 6 * 448,
  so the largest block lands on the largest E4M3 scale; g = 0 for an all-zero
  tensor.  For activations g is a static calibrated input.
* per 16-block, in correctly rounded float32 with no fused operations:
    amax = max |x_i|
    s    = (g == 0) ? 0 : fl32(fl32(amax / 6) / g)
    sb   = E4M3(s) (RNE, saturating at 448);  sv = decode(sb)
    d    = fl32(sv * g);  inv = (d == 0) ? 0 : fl32(1 / d)
    c_i  = E2M1(fl32(x_i * inv))
* packing: byte j of a row holds code 2j in its low nibble and code 2j+1 in its
  high nibble; one scale byte per block; everything row-major with K innermost.
* dequantization: x_hat = E2M1(c) * E4M3(sb) * g, in float64.

Parity unpinned by the pages: the global-scale formula and the float32 step
order are readings (the pages are silent); the tests pin everything else.
"""
from __future__ import annotations

import numpy as np

from .formats import decode_e2m1, decode_e4m3, encode_e2m1, encode_e4m3

BLOCK = 16
F32 = np.float32


def _check_finite(x: np.ndarray) -> None:
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite inputs are outside the NVFP4 contract")


def global_scale(x) -> np.float32:
    """Per-tensor decode scale g = fl32(amax|x| / 2688) of a float32 (or bf16-widened) tensor."""
    x = np.asarray(x, dtype=F32)
    _check_finite(x)
    amax = F32(np.max(np.abs(x))) if x.size else F32(0)
    return F32(amax / F32(2688.0))


def quantize(x, g) -> tuple[np.ndarray, np.ndarray]:
    """Quantize rows of x (float32 [rows, K], K % 16 == 0) with decode scale g.

    Returns (codes [rows, K] uint8 in 0..15, unpacked; scale bytes [rows, K/16] uint8).
    """
    x = np.asarray(x, dtype=F32)
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("expected [rows, K] with K a multiple of 16")
    _check_finite(x)
    g = F32(g)
    rows, K = x.shape
    xb = x.reshape(rows, K // BLOCK, BLOCK)
    amax = np.max(np.abs(xb), axis=2)                          # float32, exact
    with np.errstate(divide="ignore", invalid="ignore"):
        s = (amax / F32(6.0)).astype(F32)
        s = (s / g).astype(F32) if g != 0 else np.zeros_like(s)
    sb = encode_e4m3(s)                                        # s >= 0
    sv = decode_e4m3(sb).astype(F32)                           # exact in float32
    d = (sv * g).astype(F32)
    with np.errstate(divide="ignore"):
        inv = np.where(d == 0, F32(0), (F32(1.0) / np.where(d == 0, F32(1), d))).astype(F32)
    y = (xb * inv[:, :, None]).astype(F32)
    codes = encode_e2m1(y).reshape(rows, K)
    return codes, sb


def pack(codes) -> np.ndarray:
    """Unpacked 4-bit codes [rows, K] -> bytes [rows, K/2], even k in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack(packed) -> np.ndarray:
    """Bytes [rows, K/2] -> codes [rows, K]."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0x0F
    out[:, 1::2] = p >> 4
    return out


def quantize_packed(x, g) -> tuple[np.ndarray, np.ndarray]:
    codes, sb = quantize(x, g)
    return pack(codes), sb


def dequantize(packed, scales, g) -> np.ndarray:
    """Packed codes [rows, K/2] + scale bytes [rows, K/16] + g -> float64 [rows, K]."""
    vals = decode_e2m1(unpack(packed))
    rows, K = vals.shape
    sv = decode_e4m3(scales).astype(np.float64)
    return (vals.reshape(rows, K // BLOCK, BLOCK) * sv[:, :, None] * float(g)).reshape(rows, K)
