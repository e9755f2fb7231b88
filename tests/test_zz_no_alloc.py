"""nvfp4_gemm_scratch, the product for callers that cannot allocate (its split-K workspace is a
fixed device array inside the library), called through the C ABI: bit-identical to nvfp4_gemm_ws
with a caller workspace, on two calls in a row, the second with a smaller product, and inside a
replayed HIP graph; products the fixed array cannot hold are refused.  The shapes are the
16-node tree-verification pass of the page "TensorRT Edge-LLM Completes the MLPerf Edge Agentic
Benchmark 6.4x Faster on Jetson AGX Thor" (section "Using tree-based multi-token prediction to
accelerate LLM inference") and a smaller product of the same kind."""
import numpy as np
import pytest
import torch

import gpu_util as U
from nvfp4_w4a4_block_amd import binding as B
from oracle import gemm as G
from oracle import quant as Q

pytestmark = pytest.mark.gpu


def _operands(M, K, N, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.01).astype(np.float32)
    A = np.abs(rng.standard_normal((M, K))).astype(np.float32)
    g_a = Q.global_scale(A)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(W))
    ac, asc = B.nvfp4_quantize_act(U.dev_f32(A), U.scalar(g_a))
    return (ac, asc, U.scalar(g_a), wc, ws, gw), (A, W, g_a)


def _scratch_call(dev, M, K, N, out):
    ac, asc, ga, wc, ws, gw = dev
    return B.load().nvfp4_gemm_scratch(M, K, N, ac.data_ptr(), asc.data_ptr(), ga.data_ptr(), wc.data_ptr(),
                                       ws.data_ptr(), gw.data_ptr(), out.data_ptr(), B.NVFP4_F32,
                                       torch.cuda.current_stream().cuda_stream)


def test_scratch_matches_workspace_call_twice_then_smaller():
    U.require_gpu_lib()
    for (M, K, N), seed in (((16, 25600, 5120), 1), ((16, 12800, 2048), 2)):
        need = int(B.load().nvfp4_gemm_workspace_bytes(M, K, N))
        assert 0 < need <= B.SCRATCH_BYTES
        dev, (A, W, g_a) = _operands(M, K, N, seed)
        ws = torch.zeros((need,), dtype=torch.uint8, device=U.DEV)
        ref = B.nvfp4_gemm(*dev, out_dtype=torch.float32, workspace=ws)
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device=U.DEV)
        assert _scratch_call(dev, M, K, N, out) == B.NVFP4_OK
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), (M, K, N)
        # the result also meets the oracle's bound on a sample of columns
        cols = np.arange(0, N, 97)
        ap, asp = Q.quantize_packed(A, g_a)
        wp, wsp = Q.quantize_packed(W[cols], Q.global_scale(W))
        C, T = G.gemm_ref(ap, asp, g_a, wp, wsp, Q.global_scale(W))
        U.assert_within(out.cpu().numpy()[:, cols], C, T, f"scratch {M}x{K}x{N}")


def test_scratch_unsplit_products_and_graph_replay():
    """Products that need no workspace run as nvfp4_gemm does; the split product inside a
    replayed graph reproduces the eager result on every replay."""
    U.require_gpu_lib()
    M, K, N = 2, 5120, 3000
    dev, _ = _operands(M, K, N, 3)
    out = torch.empty((M, N), dtype=torch.float32, device=U.DEV)
    assert _scratch_call(dev, M, K, N, out) == B.NVFP4_OK
    assert torch.equal(out.view(torch.int32), B.nvfp4_gemm(*dev, out_dtype=torch.float32).view(torch.int32))
    M, K, N = 16, 25600, 1024
    dev, _ = _operands(M, K, N, 4)
    out = torch.empty((M, N), dtype=torch.float32, device=U.DEV)
    assert _scratch_call(dev, M, K, N, out) == B.NVFP4_OK
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        assert _scratch_call(dev, M, K, N, out) == B.NVFP4_OK
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        assert _scratch_call(dev, M, K, N, out) == B.NVFP4_OK
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32))


def test_scratch_validation():
    U.require_gpu_lib()
    lib = B.load()
    A16 = 0x10000
    assert lib.nvfp4_gemm_scratch(16, 24, 64, A16, A16, A16, A16, A16, A16, A16, B.NVFP4_F32, None) == \
        B.NVFP4_ERR_SHAPE
    assert lib.nvfp4_gemm_scratch(16, 256, 64, A16, A16, A16, A16, A16, A16, 0, B.NVFP4_F32, None) == \
        B.NVFP4_ERR_NULL
    assert lib.nvfp4_gemm_scratch(0, 256, 64, 0, 0, 0, 0, 0, 0, 0, B.NVFP4_F32, None) == B.NVFP4_OK
