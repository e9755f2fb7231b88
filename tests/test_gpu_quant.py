"""GPU parity of NVFP4 quantization: codes, scales and the weight tensor scale are bit-exact
against the CPU oracle (weights once offline and activations on the fly, both NVFP4 on the
page "TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x Faster on Jetson AGX
Thor", section "Using NVFP4 quantization to accelerate Qwen3.6-27B inference")."""
import os

import numpy as np
import pytest
import torch

import gpu_util as U
from nvfp4_w4a4_block_amd import binding as B
from nvfp4_w4a4_block_amd import workloads as WL
from oracle import quant as Q

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# (workload, M, K, N): reduced sizes that still span many blocks, and a K % 32 == 16 case.
SMALL = [
    ("tiny", None, None, None),
    ("decode_up", 1, 5120, 512),
    ("verify_down", 16, 25600, 48),
    ("lm_head", 16, 5120, 300),
    ("prefill", 130, 512, 272),
    ("decode_up", 3, 1040, 33),
]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    U.require_gpu_lib()


def _check_weights(W: np.ndarray, w_dev: torch.Tensor, rows=None):
    codes, scales, g = B.nvfp4_quantize_weights(w_dev)
    torch.cuda.synchronize()
    W32 = W if W.dtype == np.float32 else WL.bf16_bits_to_f32(W)
    g_ref = Q.global_scale(W32)
    assert U.f32_bits(g.item()) == U.f32_bits(g_ref), (g.item(), g_ref)
    sel = slice(None) if rows is None else rows
    p, s = Q.quantize_packed(W32[sel], g_ref)
    np.testing.assert_array_equal(codes.cpu().numpy()[sel], p)
    np.testing.assert_array_equal(scales.cpu().numpy()[sel], s)


@pytest.mark.parametrize("name,M,K,N", SMALL)
def test_quantize_weights_bitexact(name, M, K, N):
    inp = WL.generate(WL.get(name), M=M, K=K, N=N)
    _check_weights(inp.W, U.dev_f32(inp.W))


def test_quantize_weights_bf16_input():
    rng = np.random.default_rng(21)
    bits = WL.f32_to_bf16_bits((rng.standard_normal((70, 512)) * 0.02).astype(np.float32))
    _check_weights(bits, U.dev_bf16_bits(bits))


@pytest.mark.parametrize("name,M,K,N", SMALL)
def test_quantize_act_bitexact(name, M, K, N):
    inp = WL.generate(WL.get(name), M=M, K=K, N=N)
    a = inp.a_f32()
    g_a = Q.global_scale(a)
    codes, scales = B.nvfp4_quantize_act(U.dev_acts(inp), U.scalar(g_a))
    p, s = Q.quantize_packed(a, g_a)
    np.testing.assert_array_equal(codes.cpu().numpy(), p)
    np.testing.assert_array_equal(scales.cpu().numpy(), s)


def test_hand_worked_blocks_golden():
    """The GPU reproduces the hand-derived blocks of tests/golden/hand_blocks.txt directly."""
    vals, scale_bytes, packed = [], [], []
    with open(os.path.join(GOLDEN, "hand_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            _, v, g, sb, pk = [t.strip() for t in line.split(";")]
            assert float(g) == 1.0
            vals += [float(x) for x in v.split()]
            scale_bytes.append(int(sb, 16))
            packed += [int(b, 16) for b in pk.split()]
    x = np.array(vals, dtype=np.float32)[None, :]
    codes, scales = B.nvfp4_quantize_act(U.dev_f32(x), U.scalar(np.float32(1)))
    assert scales.cpu().numpy()[0].tolist() == scale_bytes
    assert codes.cpu().numpy()[0].tolist() == packed


def test_scale_extremes_and_saturation():
    """Blocks spanning 60 binades, subnormal E4M3 scales, saturated scales (g too small),
    exact E2M1 midpoints, signed zeros and all-zero blocks."""
    rng = np.random.default_rng(77)
    rows, K = 96, 256
    x = rng.standard_normal((rows, K)).astype(np.float32)
    x *= np.exp2(rng.integers(-30, 30, (rows, K // 16))).astype(np.float32).repeat(16, axis=1)
    x[5, :16] = 0.0
    x[6, :16] = -0.0
    x[7, :16] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6] * 2, np.float32) * np.float32(2.0 ** -7)
    x[8, 16:32] = np.float32(1e-38)          # fp32 subnormal-adjacent inputs
    for g in (Q.global_scale(x), np.float32(Q.global_scale(x) / 64), np.float32(2.0 ** -7), np.float32(0)):
        codes, scales = B.nvfp4_quantize_act(U.dev_f32(x), U.scalar(g))
        p, s = Q.quantize_packed(x, g)
        np.testing.assert_array_equal(scales.cpu().numpy(), s, err_msg=f"g={g}")
        np.testing.assert_array_equal(codes.cpu().numpy(), p, err_msg=f"g={g}")


def test_e2m1_decision_points():
    """Every E2M1 decision point (the midpoints .25, .75, 1.25, 1.75, 2.5, 3.5 and 5 between
    neighbouring magnitudes), one fp32 ulp on either side, both signs, signed zeros, fp32
    subnormals and values just past 6, each in a block whose largest magnitude is 6 under g = 1:
    the block scale is then exactly 1 and every value is encoded as it is (round to nearest,
    ties to the even code, saturation at 6)."""
    f32 = np.float32
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = []
    for m in mids:
        m = f32(m)
        vals += [np.nextafter(m, f32(0)), m, np.nextafter(m, f32(np.inf))]
    vals += [0.0, 1e-38, 1e-45, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    vals = np.array(vals, f32)
    vals = np.concatenate([vals, -vals, np.array([-0.0], f32)])
    blocks = []
    for i in range(0, len(vals), 15):
        blk = np.full(16, f32(0), f32)
        chunk = vals[i:i + 15]
        blk[:len(chunk)] = chunk
        blk[15] = f32(6.0)
        blocks.append(blk)
    # values past 6 in a block whose scale still rounds to 1: they saturate to code 7
    blocks.append(np.array([6.2, -6.2, 6.1, 0.3] + [0.0] * 12, f32))
    x = np.concatenate(blocks).reshape(1, -1)
    pad = (-x.shape[1]) % 64
    x = np.concatenate([x, np.zeros((1, pad), f32)], axis=1)
    g = f32(1.0)
    codes, scales = B.nvfp4_quantize_act(U.dev_f32(x), U.scalar(g))
    p, s = Q.quantize_packed(x, g)
    np.testing.assert_array_equal(scales.cpu().numpy(), s)
    np.testing.assert_array_equal(codes.cpu().numpy(), p)
    assert int(s[0, 0]) == 0x38  # E4M3 1.0: the values above were encoded unscaled


def test_zero_tensor_and_empty():
    w = torch.zeros((32, 64), dtype=torch.float32, device=U.DEV)
    codes, scales, g = B.nvfp4_quantize_weights(w)
    assert g.item() == 0.0 and not codes.any().item() and not scales.any().item()
    codes, scales, g = B.nvfp4_quantize_weights(torch.zeros((0, 64), dtype=torch.float32, device=U.DEV))
    assert g.item() == 0.0 and codes.numel() == 0
    codes, scales = B.nvfp4_quantize_act(torch.zeros((0, 64), dtype=torch.bfloat16, device=U.DEV),
                                         U.scalar(np.float32(1)))
    assert codes.numel() == 0


@pytest.mark.parametrize("name", ["decode_up", "verify_down", "lm_head", "prefill"])
def test_full_size_weights_sampled_rows(name):
    """Full-size weight matrices: tensor scale over all of W, codes/scales on sampled rows."""
    wl = WL.get(name)
    inp = WL.generate(wl)
    mats = [inp.W] + ([inp.W2] if inp.W2 is not None else [])
    for W in mats:
        rng = np.random.default_rng(1)
        rows = np.unique(np.concatenate([[0, W.shape[0] - 1], rng.choice(W.shape[0], 62, replace=False)]))
        _check_weights(W, U.dev_f32(W), rows=rows)
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["decode_up", "verify_down", "lm_head", "prefill"])
def test_full_size_acts(name):
    inp = WL.generate(WL.get(name))
    a = inp.a_f32()
    g_a = Q.global_scale(a)
    codes, scales = B.nvfp4_quantize_act(U.dev_acts(inp), U.scalar(g_a))
    p, s = Q.quantize_packed(a, g_a)
    np.testing.assert_array_equal(codes.cpu().numpy(), p)
    np.testing.assert_array_equal(scales.cpu().numpy(), s)
