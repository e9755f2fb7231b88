"""Pins of the FP8 E4M3 KV-cache codec oracle (oracle/kvfp8.py), CPU only."""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import kvfp8 as KV

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_fp8_cases.txt")


def cases():
    out = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        d, s, x, q = [f.strip() for f in line.split(";")]
        out.append((d, np.float32(float(s)), np.float32(float(x)), int(q, 16)))
    return out


@pytest.mark.parametrize("case", cases(), ids=lambda c: c[0][:40])
def test_hand_worked_elements(case):
    _, s, x, q = case
    assert int(KV.encode(np.array([x]), s)[0]) == q


def test_every_code_round_trips_under_power_of_two_scales():
    codes = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    for e in range(-12, 13):
        s = np.float32(2.0 ** e)
        x = KV.decode_f32(codes, s)                      # exact: a power-of-two scale
        np.testing.assert_array_equal(x.astype(np.float64), F.decode_e4m3(codes) * 2.0 ** e)
        np.testing.assert_array_equal(KV.encode(x, s), codes)


def test_encode_matches_torch_float8_within_range():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(200000) * 50, rng.standard_normal(50000) * 1e-3,
                        (F.decode_e4m3(np.arange(0x7E)) + F.decode_e4m3(np.arange(1, 0x7F))) / 2]).astype(np.float32)
    s = np.float32(0.37)
    y = (x * np.float32(np.float32(1) / s)).astype(np.float32)
    keep = np.abs(y) <= 448  # torch's cast turns overflow into NaN; the codec saturates (pinned below)
    ref = torch.from_numpy(y[keep]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(KV.encode(x[keep], s), ref)
    assert np.all(KV.encode(np.array([1e6, -1e6, 480.0 * 0.37], dtype=np.float32), s) == [0x7E, 0xFE, 0x7E])


def test_decode_matches_torch_and_error_bound():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(100000) * 3).astype(np.float32)
    s = KV.calibrated_scale(x)
    q = KV.encode(x, s)
    xf = KV.decode_f32(q, s)
    ref = (torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float32) * float(s)).numpy()
    np.testing.assert_array_equal(xf, ref)
    # half a step of the 3-bit mantissa: |x_hat - x| <= 2^-4 |x| for normal codes, <= 2^-10 s for subnormal ones
    y = np.abs(x.astype(np.float64) / float(s))
    bound = np.where(y >= 2.0 ** -6, 2.0 ** -4 * np.abs(x.astype(np.float64)), 2.0 ** -10 * float(s)) * 1.0001
    assert np.all(np.abs(xf.astype(np.float64) - x) <= bound + 1e-30)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(KV.f32_to_bf16_bits(v), ref)


def test_calibrated_scale():
    assert KV.calibrated_scale(np.array([0.0, -896.0, 3.0])) == np.float32(2.0)
    assert KV.calibrated_scale(np.zeros(4)) == 0
