"""GPU parity of the FP8 E4M3 KV-cache codec (nvfp4_kv_fp8_encode / _decode) against the oracle:
codes and decoded values bit for bit (integer and exactly specified fp32 work).  Page "TensorRT
Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x Faster on Jetson AGX Thor", section "Using
NVFP4 quantization to accelerate Qwen3.6-27B inference" (the KV cache is FP8)."""
import numpy as np
import pytest
import torch

import gpu_util as U
from nvfp4_w4a4_block_amd import binding as B
from nvfp4_w4a4_block_amd import workloads as WL
from oracle import formats as F
from oracle import kvfp8 as KV

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    U.require_gpu_lib()


def check(x_f32: np.ndarray, s, dtype):
    """x_f32 holds the exact values handed to the GPU (bf16-representable when dtype is bf16)."""
    if dtype == torch.bfloat16:
        x = U.dev_bf16_bits(KV.f32_to_bf16_bits(x_f32))
    else:
        x = U.dev_f32(x_f32)
    sd = U.scalar(np.float32(s))
    q = B.nvfp4_kv_fp8_encode(x, sd)
    y32 = B.nvfp4_kv_fp8_decode(q, sd, torch.float32)
    y16 = B.nvfp4_kv_fp8_decode(q, sd, torch.bfloat16)
    torch.cuda.synchronize()
    q_ref = KV.encode(x_f32, s)
    np.testing.assert_array_equal(U.host(q).reshape(-1), q_ref.reshape(-1))
    np.testing.assert_array_equal(np.ascontiguousarray(U.host(y32), dtype=np.float32).view(np.uint32).reshape(-1),
                                  KV.decode_f32(q_ref, s).view(np.uint32).reshape(-1))
    y16_bits = y16.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    np.testing.assert_array_equal(y16_bits, KV.decode_bf16_bits(q_ref, s).reshape(-1))


@pytest.mark.parametrize("n", [1, 15, 16, 17, 1000, 65543, 4096 * 256 + 3, 4096 * 256 * 5 + 16])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_encode_decode_match_oracle(n, dtype):
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * 4).astype(np.float32)
    if dtype == torch.bfloat16:
        x = WL.bf16_bits_to_f32(KV.f32_to_bf16_bits(x))
    check(x, KV.calibrated_scale(x), dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_special_values_and_scales(dtype):
    codes = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    vals = F.decode_e4m3(codes)
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([vals, mids, [0.0, -0.0, 1e6, -1e6, 460.0, -470.0, 2.0 ** -12, -(2.0 ** -11)]])
    x = x.astype(np.float32)
    if dtype == torch.bfloat16:
        x = WL.bf16_bits_to_f32(KV.f32_to_bf16_bits(x))
    for s in (1.0, 0.25, 3.0, 0.0, 1.7e-3):
        check(x, np.float32(s), dtype)


def test_empty_is_a_no_op():
    sd = U.scalar(np.float32(1.0))
    q = B.nvfp4_kv_fp8_encode(torch.empty(0, dtype=torch.bfloat16, device="cuda"), sd)
    assert q.numel() == 0
    assert B.nvfp4_kv_fp8_decode(q, sd).numel() == 0


def test_full_layer_kv():
    """One layer's K and V for a 23,552-token context (8 heads x 128), the benchmark's size."""
    bits = WL.make_kv()
    x = WL.bf16_bits_to_f32(bits).reshape(-1)
    check(x, KV.calibrated_scale(x), torch.bfloat16)
