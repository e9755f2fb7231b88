"""The persistent M <= 16 weight stream (gemm_m16_stream_kernel) against the CPU oracle.

The kernel serves the language-model head over the 16 nodes of a verification tree (page
"TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x Faster on Jetson AGX Thor",
section "Using tree-based multi-token prediction to accelerate LLM inference").  Its structure
adds cases of its own: K walked in chunks of 20, 16, 12 or 8 lines (one or several chunks),
waves that own no group, one group or several, ragged last groups, M below 16, and more
workgroups than CUs for very tall matrices.  Weights here are random NVFP4 codes and E4M3
scale bytes (every code, moderate scales), so tall shapes need no float quantization; the
oracle dequantizes exactly those bytes.  Bar: |gpu - C| <= 1e-3 * sum_k |a_hat * w_hat| (plus
the bf16 rounding of a bf16 result), C the oracle's fp64 product; results bit-identical from
call to call.
"""
import numpy as np
import pytest
import torch

import gpu_util as U
from nvfp4_w4a4_block_amd import binding as B
from oracle import gemm as G
from oracle import quant as Q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    U.require_gpu_lib()


def _operands(M, K, N, seed):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K)).astype(np.float32)
    g_a = Q.global_scale(A)
    ac, asc = B.nvfp4_quantize_act(U.dev_f32(A), U.scalar(g_a))
    ap, asp = Q.quantize_packed(A, g_a)
    wp = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    wsp = rng.integers(0x28, 0x48, (N, K // 16), dtype=np.uint8)  # E4M3 2^-2 .. 2^1.875
    g_w = np.float32(0.0173)
    dev = (ac, asc, U.scalar(g_a), torch.from_numpy(wp).to(U.DEV), torch.from_numpy(wsp).to(U.DEV),
           U.scalar(g_w))
    return dev, (ap, asp, g_a, wp, wsp, g_w)


# (M, K, N): chunk length C and chunk count, groups per wave (256 CUs x 8 waves)
CASES = [
    (16, 5120, 4100),    # C = 20, 2 chunks; ragged last group; most waves own 1 group or none
    (5, 4096, 1000),     # C = 16, 2 chunks, M < 16
    (16, 3072, 777),     # C = 12, 2 chunks
    (3, 1024, 333),      # C = 8, 1 chunk
    (16, 25600, 600),    # C = 20, 10 chunks
    (1, 2048, 16),       # one group in all: every other wave owns none
    (16, 6144, 2000),    # C = 16, 3 chunks
    (9, 2560, 65600),    # 4100 groups: 2-3 per wave
]


@pytest.mark.parametrize("M,K,N", CASES)
def test_stream_kernel_matches_oracle(M, K, N):
    dev, host = _operands(M, K, N, 11 * M + K + 3 * N)
    C, T = G.gemm_ref(*host)
    for out_dtype in (torch.float32, torch.bfloat16):
        o1 = B.nvfp4_gemm(*dev, out_dtype=out_dtype, path=B.KERNEL_M16_STREAM)
        o2 = B.nvfp4_gemm(*dev, out_dtype=out_dtype, path=B.KERNEL_M16_STREAM)
        assert torch.equal(o1.view(torch.uint8), o2.view(torch.uint8)), "not deterministic"
        U.assert_within(U.host(o1), C, T + U.out_rounding_slack(C, out_dtype), f"{(M, K, N)} {out_dtype}")


def test_stream_kernel_tall_matrix_more_workgroups_than_cus():
    """4 x 1024 x 300000: 18750 groups, more than 8 per wave of one workgroup per CU, so the
    grid grows past the CU count; sampled columns (the first and last groups among them)."""
    M, K, N = 4, 1024, 300000
    dev, (ap, asp, g_a, wp, wsp, g_w) = _operands(M, K, N, 5)
    rng = np.random.default_rng(6)
    cols = np.unique(np.concatenate([np.arange(32), np.arange(N - 32, N), rng.integers(0, N, 512)]))
    C, T = G.gemm_ref(ap, asp, g_a, wp[cols], wsp[cols], g_w)
    out = U.host(B.nvfp4_gemm(*dev, out_dtype=torch.float32, path=B.KERNEL_M16_STREAM))
    U.assert_within(out[:, cols], C, T, "tall")


def test_stream_kernel_agrees_with_m_tile_within_bound_at_lm_head_rows():
    """16 x 5120 x 70000 through the automatic dispatch (which names the stream kernel) and
    through the M-tile kernel: both within the bound of the oracle on sampled columns."""
    M, K, N = 16, 5120, 70000
    assert B.gemm_dispatch(M, K, N, 0) == B.KERNEL_M16_STREAM
    dev, (ap, asp, g_a, wp, wsp, g_w) = _operands(M, K, N, 8)
    rng = np.random.default_rng(9)
    cols = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N), rng.integers(0, N, 400)]))
    C, T = G.gemm_ref(ap, asp, g_a, wp[cols], wsp[cols], g_w)
    auto = U.host(B.nvfp4_gemm(*dev, out_dtype=torch.float32))
    tile = U.host(B.nvfp4_gemm(*dev, out_dtype=torch.float32, path=B.KERNEL_M16))
    U.assert_within(auto[:, cols], C, T, "auto (stream)")
    U.assert_within(tile[:, cols], C, T, "M-tile")
