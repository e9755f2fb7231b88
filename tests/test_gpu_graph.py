"""The benchmark replays the decode step (activation quantization + GEMV) as a HIP graph:
every replay must reproduce the eager result bit for bit, with eager work and
synchronizations between replays."""
import numpy as np
import pytest
import torch

import gpu_util as U
from nvfp4_w4a4_block_amd import binding as B
from nvfp4_w4a4_block_amd import workloads as WL
from oracle import quant as Q

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N", [(1, 5120, 2048), (16, 2560, 1024), (160, 1024, 384)])
def test_graph_replays_match_eager(M, K, N):
    U.require_gpu_lib()
    inp = WL.generate(WL.get("decode_up"), M=M, K=K, N=N)
    g_a = U.scalar(Q.global_scale(inp.a_f32()))
    a = U.dev_acts(inp)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(inp.W))
    ac = torch.empty((M, K // 2), dtype=torch.uint8, device=U.DEV)
    asc = torch.empty((M, K // 16), dtype=torch.uint8, device=U.DEV)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=U.DEV)

    def step():
        B.nvfp4_quantize_act(a, g_a, ac, asc)
        B.nvfp4_gemm(ac, asc, g_a, wc, ws, gw, out=out)

    step()
    torch.cuda.synchronize()
    eager = (ac.clone(), asc.clone(), out.clone())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        ac.zero_(); asc.zero_(); out.zero_()          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((ac, asc, out), eager):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {r} differs"


@pytest.mark.parametrize("M,K,N", [(1, 5120, 2048), (2, 4096, 1000), (3, 2048, 500)])
def test_dynamic_scale_step_graph_replays(M, K, N):
    """The decode step with the tensor scale computed on the device (one fused kernel for one or
    two rows, the scale kernel and the quantized GEMM otherwise): every replay reproduces g_a,
    the activation codes and the output of the eager call."""
    U.require_gpu_lib()
    inp = WL.generate(WL.get("decode_up"), M=M, K=K, N=N)
    a = U.dev_acts(inp)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(inp.W))
    ac = torch.empty((M, K // 2), dtype=torch.uint8, device=U.DEV)
    asc = torch.empty((M, K // 16), dtype=torch.uint8, device=U.DEV)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=U.DEV)
    g_a = torch.empty((1,), dtype=torch.float32, device=U.DEV)

    def step():
        B.nvfp4_quantize_gemm_dynamic(a, wc, ws, gw, out=out, a_codes=ac, a_scales=asc, g_a=g_a)

    step()
    torch.cuda.synchronize()
    eager = (g_a.clone(), ac.clone(), asc.clone(), out.clone())
    assert U.f32_bits(g_a.item()) == U.f32_bits(Q.global_scale(inp.a_f32()))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        g_a.fill_(-1.0); ac.zero_(); asc.zero_(); out.zero_()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((g_a, ac, asc, out), eager):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {r} differs"
