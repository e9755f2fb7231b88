"""The seeded synthetic inputs have the structure each workload states (CPU only)."""
import numpy as np

from nvfp4_w4a4_block_amd import workloads as WL


def test_deterministic_and_small_override():
    wl = WL.get("decode_up")
    a = WL.generate(wl, M=2, K=512, N=64)
    b = WL.generate(wl, M=2, K=512, N=64)
    assert np.array_equal(a.W, b.W) and np.array_equal(a.A, b.A)
    assert a.W.dtype == np.float32 and a.W.shape == (64, 512)
    assert a.A.dtype == np.uint16 and a.A.shape == (2, 512)


def test_outlier_channels():
    wl = WL.get("decode_up")
    inp = WL.generate(wl, M=4, K=5120, N=16)
    a = inp.a_f32()
    big = np.abs(a) > 8          # N(0,1) essentially never exceeds 8; x20 outliers usually do
    cols = np.nonzero(big.any(axis=0))[0]
    assert 0 < cols.size <= 26    # round(0.005 * 5120) outlier channels, shared by all rows


def test_abs_and_zero_fraction():
    wl = WL.get("verify_down")
    inp = WL.generate(wl, M=16, K=2560, N=16)
    a = inp.a_f32()
    assert np.all(a >= 0)
    assert int((a == 0).sum()) == round(0.01 * 16 * 2560)


def test_prefill_has_chained_weights():
    wl = WL.get("prefill")
    inp = WL.generate(wl, M=8, K=64, N=96)
    assert inp.W.shape == (96, 64) and inp.W2.shape == (64, 96)


def test_workload_byte_counts():
    assert WL.get("decode_up").weight_bytes == 73_728_000
    assert WL.get("verify_down").weight_bytes == 73_728_000
    assert WL.get("lm_head").weight_bytes == 437_575_680
    assert WL.get("tiny").weight_bytes == 36_864
