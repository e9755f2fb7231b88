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


@pytest.mark.parametrize("M,K,N", [(1, 5120, 2048), (16, 2560, 1024), (16, 5120, 70000), (160, 1024, 384)])
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


@pytest.mark.parametrize("N", [20000, 70000])
def test_tree_verify_graph_replays(N):
    """The LM head with the fused argmax and the acceptance kernel inside a replayed HIP graph
    (20000 rows: the M-tile kernel; 70000: the persistent stream): the argmax key slots return
    to zero after every call, so every replay reproduces the eager greedy tokens and acceptance
    (with eager work between replays)."""
    U.require_gpu_lib()
    M, K = 16, 5120
    inp = WL.generate(WL.get("lm_head"), M=M, K=K, N=N)
    g_a = U.scalar(Q.global_scale(inp.a_f32()))
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(inp.W))
    ac, asc = B.nvfp4_quantize_act(U.dev_acts(inp), g_a)
    parent, chain = [-1], [0]
    for _ in range(7):
        parent += [chain[-1], chain[-1]]
        chain.append(len(parent) - 2)
    parent.append(chain[-1])
    parent_d = torch.tensor(parent, dtype=torch.int32, device=U.DEV)
    keys = torch.zeros((1024,), dtype=torch.int64, device=U.DEV)
    greedy0, _, _ = B.nvfp4_tree_verify(ac, asc, g_a, wc, ws, gw, parent_d,
                                        torch.zeros(M, dtype=torch.int32, device=U.DEV), keys=keys)
    # drafts that follow the greedy chain for a few nodes
    g0 = greedy0.cpu().numpy()
    draft = [0] + [int(g0[parent[v]]) if v < 8 else 0 for v in range(1, M)]
    draft_d = torch.tensor(draft, dtype=torch.int32, device=U.DEV)
    greedy = torch.empty((M,), dtype=torch.int32, device=U.DEV)
    result = torch.empty((3 + M,), dtype=torch.int32, device=U.DEV)
    lib = B.load()

    def call():
        st = lib.nvfp4_tree_verify(M, K, N, ac.data_ptr(), asc.data_ptr(), g_a.data_ptr(), wc.data_ptr(),
                                   ws.data_ptr(), gw.data_ptr(), parent_d.data_ptr(), draft_d.data_ptr(), None,
                                   greedy.data_ptr(), result.data_ptr(), keys.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
        assert st == 0

    call()
    torch.cuda.synchronize()
    eager = (greedy.clone(), result.clone())
    assert torch.equal(eager[0], greedy0)
    assert not keys.any().item()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        call()
    for r in range(4):
        greedy.fill_(-5); result.fill_(-5)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(greedy, eager[0]) and torch.equal(result, eager[1]), f"replay {r} differs"
        assert not keys.any().item()
