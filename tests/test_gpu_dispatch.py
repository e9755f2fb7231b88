"""Every kernel of the product against the CPU oracle, reached two ways: through the automatic
dispatch (nvfp4_gemm_dispatch names the kernel a shape runs, and the result is checked), and
by selecting the kernel explicitly (nvfp4_gemm_ex's kernel selectors) on shapes it takes.

The shapes stand in for the products of the page "TensorRT Edge-LLM Completes the MLPerf Edge
Agentic Benchmark 6.4x Faster on Jetson AGX Thor": one or two decode rows (section "Using NVFP4
quantization to accelerate Qwen3.6-27B inference"), the 16 rows of a verification tree (section
"Using tree-based multi-token prediction to accelerate LLM inference") and a suffix prefill
(section "Reusing KV cache across agent turns").  Bar: |gpu - C| <= 1e-3 * sum_k |a_hat * w_hat|
(plus the bf16 rounding of a bf16 result), C the oracle's fp64 product.
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
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = rng.standard_normal((M, K)).astype(np.float32)
    g_a, g_w = Q.global_scale(A), Q.global_scale(W)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(W))
    ac, asc = B.nvfp4_quantize_act(U.dev_f32(A), U.scalar(g_a))
    ap, asp = Q.quantize_packed(A, g_a)
    wp, wsp = Q.quantize_packed(W, g_w)
    C, T = G.gemm_ref(ap, asp, g_a, wp, wsp, g_w)
    return (ac, asc, U.scalar(g_a), wc, ws, gw), C, T


# (M, K, N, workspace?) -> the kernel the automatic dispatch runs
AUTO = [
    ((1, 5120, 700, False), B.KERNEL_GEMV_FP4),     # decode: K % 1024 == 0, K <= 8192
    ((2, 1024, 300, False), B.KERNEL_GEMV_FP4),
    ((1, 25600, 640, False), B.KERNEL_GEMV_FLAT),   # decode down-projection: long K
    ((2, 2560, 333, False), B.KERNEL_GEMV_FLAT),
    ((1, 512, 100, False), B.KERNEL_SKINNY256),     # short K, no FP4 / flat kernel
    ((1, 1040, 77, False), B.KERNEL_SKINNY16),      # K % 256 != 0
    ((16, 25600, 1024, False), B.KERNEL_SKINNY256), # starved and long K without a workspace
    ((16, 25600, 1024, True), B.KERNEL_M16),        # ... split with one
    ((16, 5120, 20000, False), B.KERNEL_M16),       # enough rows: unsplit
    ((3, 1024, 65536, False), B.KERNEL_M16_STREAM), # a tall matrix: 2 groups of 16 rows per wave
    ((16, 5120, 3000, True), B.KERNEL_SKINNY256),   # short K, N <= 16384: no workspace needed
    ((7, 1040, 300, False), B.KERNEL_SKINNY16),
    ((17, 1024, 300, False), B.KERNEL_TILED_PERSISTENT),
    ((129, 768, 200, False), B.KERNEL_TILED),
]


@pytest.mark.parametrize("shape,kernel", AUTO, ids=lambda v: str(v))
def test_auto_dispatch_names_and_matches(shape, kernel):
    M, K, N, with_ws = shape
    need = int(B.load().nvfp4_gemm_workspace_bytes(M, K, N)) if with_ws else 0
    assert B.gemm_dispatch(M, K, N, need) == kernel, B.KERNEL_NAMES[B.gemm_dispatch(M, K, N, need)]
    dev, C, T = _operands(M, K, N, M + 3 * K + 7 * N)
    ws = torch.zeros((need,), dtype=torch.uint8, device=U.DEV) if need else None
    for out_dtype in (torch.float32, torch.bfloat16):
        out = B.nvfp4_gemm(*dev, out_dtype=out_dtype, workspace=ws) if ws is not None else \
            B.nvfp4_gemm(*dev, out_dtype=out_dtype)
        U.assert_within(U.host(out), C, T + U.out_rounding_slack(C, out_dtype),
                        f"{shape} {B.KERNEL_NAMES[kernel]} {out_dtype}")


def test_auto_dispatch_covers_every_kernel():
    assert {k for _, k in AUTO} == set(B.KERNEL_NAMES)


# Each kernel selected explicitly: a ragged shape it takes, and one it refuses.
FORCED = [
    (B.KERNEL_GEMV_FP4, (2, 3072, 515), (3, 3072, 515)),
    (B.KERNEL_GEMV_FLAT, (1, 4352, 1001), (1, 1024, 100)),
    (B.KERNEL_M16, (13, 1152, 257), (17, 1152, 257)),
    (B.KERNEL_M16_STREAM, (13, 2560, 1000), (4, 1152, 257)),
    (B.KERNEL_SKINNY256, (33, 768, 129), (4, 784, 129)),
    (B.KERNEL_SKINNY16, (20, 784, 129), None),
    (B.KERNEL_TILED_PERSISTENT, (40, 2048, 170), (40, 1280, 170)),
    (B.KERNEL_TILED, (5, 784, 129), None),
]


@pytest.mark.parametrize("kernel,good,bad", FORCED, ids=lambda v: B.KERNEL_NAMES.get(v, str(v)))
def test_forced_kernel(kernel, good, bad):
    M, K, N = good
    dev, C, T = _operands(M, K, N, 5 * M + K + N)
    for out_dtype in (torch.float32, torch.bfloat16):
        out = B.nvfp4_gemm(*dev, out_dtype=out_dtype, path=kernel)
        U.assert_within(U.host(out), C, T + U.out_rounding_slack(C, out_dtype),
                        f"{B.KERNEL_NAMES[kernel]} {good} {out_dtype}")
    if bad is not None:
        M, K, N = bad
        dev, _, _ = _operands(M, K, N, 1)
        with pytest.raises(B.NVFP4Error) as e:
            B.nvfp4_gemm(*dev, out_dtype=torch.float32, path=kernel)
        assert e.value.status == B.NVFP4_ERR_SHAPE


def test_kernels_agree_on_a_shape_all_take():
    """A 2 x 4096 x 600 product taken by every kernel: all results within the bound, and the
    two summation orders of each kernel deterministic from call to call."""
    M, K, N = 2, 4096, 600
    dev, C, T = _operands(M, K, N, 77)
    for kernel in B.KERNEL_NAMES:
        o1 = B.nvfp4_gemm(*dev, out_dtype=torch.float32, path=kernel).cpu().numpy()
        o2 = B.nvfp4_gemm(*dev, out_dtype=torch.float32, path=kernel).cpu().numpy()
        assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32)), B.KERNEL_NAMES[kernel]
        U.assert_within(o1, C, T, B.KERNEL_NAMES[kernel])
