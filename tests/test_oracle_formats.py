"""Pins for the oracle's E2M1 / E4M3 codecs (CPU only).

Each test checks the oracle against something other than itself: the minifloat
closed form, torch's float8_e4m3fn casts (a library routine), hand-derived
rounding decisions (tests/golden/e2m1_rounding.txt) and exact rational brute force.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def minifloat_value(code: int, ebits: int, mbits: int, bias: int) -> Fraction:
    """Closed form of a sign/exponent/mantissa minifloat with subnormals (no NaN handling)."""
    s = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        v = Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
    else:
        v = (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)
    return -v if s else v


def test_e2m1_decode_matches_minifloat_closed_form():
    got = F.decode_e2m1(np.arange(16))
    for c in range(16):
        assert Fraction(got[c]) == minifloat_value(c, 2, 1, 1), c
    # the value set named by the format
    assert sorted(set(np.abs(got))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e4m3_decode_matches_closed_form_and_torch():
    b = np.arange(256)
    got = F.decode_e4m3(b)
    lib = torch.tensor(b, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for i in range(256):
        if (i & 0x7F) == 0x7F:
            assert np.isnan(got[i]) and np.isnan(lib[i])
            continue
        assert got[i] == lib[i], hex(i)
        assert Fraction(got[i]) == minifloat_value(i, 4, 3, 7), hex(i)
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_roundtrip_every_finite_byte():
    b = np.array([i for i in range(256) if (i & 0x7F) != 0x7F])
    assert np.array_equal(F.encode_e4m3(F.decode_e4m3(b)), b.astype(np.uint8))


def _e4m3_probe_values():
    """Every midpoint between adjacent non-negative E4M3 values, +-1 float32 ulp, plus spot values."""
    pos = F.decode_e4m3(np.arange(0x7F))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals = [pos.astype(np.float32), mids, np.nextafter(mids, np.float32(np.inf)),
            np.nextafter(mids, np.float32(0))]
    rng = np.random.default_rng(123)
    vals.append((rng.random(20000) * 464).astype(np.float32))
    vals.append((rng.random(20000) * 2.0 ** -5).astype(np.float32))
    vals.append(np.array([1.0625, 1.1875, 2.0 ** -10, 1.5 * 2.0 ** -10, 7 / 6, 1 / 6, 0.01 / 6,
                          448, 456, 464, 1e-40, 0.0], dtype=np.float32))
    v = np.concatenate(vals)
    return v[(v >= 0) & (v <= 464)]


def test_e4m3_encode_matches_torch_rne_on_0_to_464():
    v = _e4m3_probe_values()
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.encode_e4m3(v)
    bad = np.nonzero(got != lib)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(lib[i])) for i in bad[:10]]


def test_e4m3_spot_values():
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 1.5 * 2.0 ** -10: 0x01,
             7 / 6: 0x39, 1 / 6: 0x23, 0.01 / 6: 0x01, 448: 0x7E, 456: 0x7E, 464: 0x7E}
    for x, b in cases.items():
        assert F.encode_e4m3(np.float32(x)) == b, x


def test_e4m3_saturates_instead_of_nan():
    # torch's cast turns these into NaN (0x7F); NVFP4 scales saturate to the largest finite value.
    v = np.array([464.00003, 470, 500, 1e6, 3e38], dtype=np.float32)
    assert np.all(F.encode_e4m3(v) == 0x7E)
    assert np.all(F.encode_e4m3(-v) == 0xFE)
    with pytest.raises(ValueError):
        F.encode_e4m3(np.float32(np.nan))


def _golden_e2m1():
    rows = []
    with open(os.path.join(GOLDEN, "e2m1_rounding.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, code = [t.strip() for t in line.split(";")]
            if lhs.startswith("up ") or lhs.startswith("dn "):
                x = np.float32(float(lhs[3:]))
                toward = np.float32(np.inf) if lhs.startswith("up") else np.float32(0)
                x = np.nextafter(x, toward)
            else:
                x = np.float32(float(lhs))
            rows.append((x, int(code, 16)))
    return rows


def test_e2m1_rounding_golden():
    rows = _golden_e2m1()
    assert len(rows) >= 20
    for x, code in rows:
        assert int(F.encode_e2m1(x)) == code, (float(x), code)


def test_e2m1_roundtrip_every_code():
    c = np.arange(16)
    assert np.array_equal(F.encode_e2m1(F.decode_e2m1(c)), c.astype(np.uint8))


def test_e2m1_encode_exact_bruteforce():
    """Nearest E2M1 value by exact rational distance over all 16 codes (ties -> even mantissa)."""
    table = [(minifloat_value(c, 2, 1, 1), c) for c in range(16)]
    rng = np.random.default_rng(7)
    xs = np.concatenate([rng.uniform(-8, 8, 3000).astype(np.float32),
                         np.arange(-28, 29, dtype=np.float32) / 4])  # every quarter incl. midpoints
    got = F.encode_e2m1(xs)
    for x, g in zip(xs, got):
        fx = Fraction(float(x))
        fx_c = max(min(fx, Fraction(6)), Fraction(-6))
        best = min(abs(fx_c - v) for v, _ in table)
        cands = [c for v, c in table if abs(fx_c - v) == best]
        if len(cands) > 1:   # exact tie (or +-0): keep the candidates with the input's sign, even mantissa
            sign = 8 if np.signbit(x) else 0
            same = [c for c in cands if (c & 8) == sign] or cands
            cands = [c for c in same if (c & 1) == 0] or same
        assert int(g) in cands and len(cands) == 1, (float(x), int(g), cands)


def test_e2m1_sign_of_zero_and_nan():
    assert F.encode_e2m1(np.float32(-0.0)) == 8
    assert F.encode_e2m1(np.float32(0.0)) == 0
    assert F.encode_e2m1(np.float32(-1e-30)) == 8
    with pytest.raises(ValueError):
        F.encode_e2m1(np.float32(np.nan))
