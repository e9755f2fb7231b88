"""GPU parity of the weight-streaming GEMM for 3..16 activation rows (a line of 16 weight rows
per matrix-core tile, activations staged in LDS, the contraction optionally split over
workgroups through a caller-owned workspace) against the CPU oracle.

The shapes stand in for the 16-node tree verification pass of the page "TensorRT Edge-LLM
Completes the MLPerf Edge Agentic Benchmark 6.4x Faster on Jetson AGX Thor" (section "Using
tree-based multi-token prediction to accelerate LLM inference"): few activation rows against
long rows of NVFP4 weights.  Bar: |gpu - C| <= 1e-3 * sum_k |a_hat * w_hat| per output (plus
the bf16 rounding of the stored value), C the oracle's fp64 product; the split path must be
bit-identical from run to run and leave its counters at zero.
"""
import os

import numpy as np
import pytest
import torch

import gpu_util as U
from nvfp4_w4a4_block_amd import binding as B
from oracle import gemm as G
from oracle import quant as Q

pytestmark = pytest.mark.gpu

KNOBS = ("NVFP4_M16_G", "NVFP4_M16_RB", "NVFP4_M16_KS", "NVFP4_M16_KZ", "NVFP4_M16_D", "NVFP4_M16_CP",
         "NVFP4_M16_AW", "NVFP4_M16_SB", "NVFP4_M16_SMALL")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    U.require_gpu_lib()


@pytest.fixture()
def knobs():
    """Sets launch-plan knobs for one test and clears them afterwards."""
    set_ = {}

    def apply(**kv):
        for k, v in kv.items():
            os.environ[f"NVFP4_M16_{k}"] = str(v)
            set_[k] = v
    yield apply
    for k in KNOBS:
        os.environ.pop(k, None)


def _pair(M, K, N, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = np.abs(rng.standard_normal((M, K))).astype(np.float32)  # non-negative, as after SiLU
    A[rng.random((M, K)) < 0.01] = 0.0
    g_a = Q.global_scale(A)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(W))
    ac, asc = B.nvfp4_quantize_act(U.dev_f32(A), U.scalar(g_a))
    g_w = Q.global_scale(W)
    ap, asp = Q.quantize_packed(A, g_a)
    wp, wsp = Q.quantize_packed(W, g_w)
    C, T = G.gemm_ref(ap, asp, g_a, wp, wsp, g_w)
    return (ac, asc, U.scalar(g_a), wc, ws, gw), C, T


# (M, K, N): one line (K = 128), odd line counts, the largest K staged whole (49 lines), K
# beyond that (split required, else the older kernels), N of 1, ragged and several row blocks.
CASES = [(3, 128, 1), (5, 384, 37), (16, 1024, 300), (7, 2688, 129), (16, 6272, 64), (16, 6400, 100),
         (16, 9216, 1000), (11, 25600, 300), (16, 5120, 3000), (4, 640, 2049)]


@pytest.mark.parametrize("small", [1, 0], ids=["dispatch", "m16-forced"])
@pytest.mark.parametrize("M,K,N", CASES)
def test_m16_with_and_without_workspace(M, K, N, small, knobs):
    """small=1: the library's dispatch (short-K products with N <= 16384 run the skinny kernel);
    small=0: the M-tile kernel for every shape it supports."""
    knobs(SMALL=small)
    dev, C, T = _pair(M, K, N, 11 * M + K + N)
    for i, ws in enumerate((None, "auto")):
        out_dtype = torch.float32 if i == 0 else torch.bfloat16
        out = B.nvfp4_gemm(*dev, out_dtype=out_dtype, workspace=ws)
        U.assert_within(U.host(out), C, T + U.out_rounding_slack(C, out_dtype), f"M={M} K={K} N={N} ws={ws}")


# Launch plans forced through the tuning knobs: row groups per wave (G), row blocks (RB) and K
# slices (KS) per workgroup, K splits over workgroups (KZ), loads in flight (D), cache policy
# (CP), activations dequantized once per workgroup into a shared f16 window (AW), weight scales
# of the whole K range staged once per wave (SB).
PLANS = [dict(G=1, RB=1, KS=1, KZ=1, D=1), dict(G=4, RB=2, KS=4, KZ=1, D=2), dict(G=2, RB=1, KS=8, KZ=3, D=2),
         dict(G=1, RB=8, KS=1, KZ=7, D=4, CP=0), dict(G=4, RB=1, KS=2, KZ=13, D=1), dict(G=2, RB=4, KS=2, KZ=40, D=2, CP=2),
         dict(G=1, RB=8, KS=1, KZ=1, D=4), dict(G=1, RB=16, KS=1, KZ=5, D=2), dict(G=1, RB=8, KS=2, KZ=2, D=1),
         dict(G=1, RB=8, KS=1, KZ=1, D=2, AW=1), dict(G=1, RB=8, KS=1, KZ=3, D=1, AW=1),
         dict(G=1, RB=8, KS=1, KZ=7, D=4, AW=1), dict(G=1, RB=8, KS=1, KZ=1, D=2, AW=1, SB=1),
         dict(G=1, RB=8, KS=1, KZ=3, D=1, AW=1, SB=1), dict(G=1, RB=8, KS=1, KZ=5, D=4, AW=1, SB=1)]


@pytest.mark.parametrize("plan", PLANS, ids=lambda p: "-".join(f"{k}{v}" for k, v in p.items()))
@pytest.mark.parametrize("M,K,N", [(16, 5120, 700), (9, 3456, 333)])
def test_m16_forced_plans(M, K, N, plan, knobs):
    knobs(SMALL=0, **plan)
    dev, C, T = _pair(M, K, N, 3 * M + K + N)
    out = B.nvfp4_gemm(*dev, out_dtype=torch.float32, workspace="auto")
    U.assert_within(U.host(out), C, T, f"M={M} K={K} N={N} plan={plan}")


def test_m16_split_deterministic_and_counters_reset(knobs):
    knobs(KZ=25)
    M, K, N = 16, 25600, 512
    dev, C, T = _pair(M, K, N, 5)
    need = int(B.load().nvfp4_gemm_workspace_bytes(M, K, N))
    assert need > 0
    ws = torch.zeros((need,), dtype=torch.uint8, device=U.DEV)
    outs = [B.nvfp4_gemm(*dev, out_dtype=torch.float32, workspace=ws).cpu().numpy() for _ in range(3)]
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    U.assert_within(outs[0], C, T, "split K")
    assert not ws[:256].any().item(), "arrival counters not reset"
    # a workspace one byte short runs the unsplit kernels: same tolerance, no workspace writes
    small = torch.zeros((need - 1,), dtype=torch.uint8, device=U.DEV)
    U.assert_within(B.nvfp4_gemm(*dev, out_dtype=torch.float32, workspace=small).cpu().numpy(), C, T, "short ws")
    assert not small.any().item()


def test_m16_split_reads_fresh_partials(knobs):
    """Two different products through one workspace, alternately: every result must match its
    own oracle, so the last workgroup of a row block never adds partial sums left over from the
    other product (or from an earlier call) instead of the ones just written."""
    knobs(KZ=10)
    M, K, N = 16, 25600, 777
    dev1, C1, T1 = _pair(M, K, N, 21)
    dev2, C2, T2 = _pair(M, K, N, 22)
    ws = B.gemm_workspace(M, K, N, torch.device(U.DEV))
    assert ws is not None
    for _ in range(3):
        o1 = B.nvfp4_gemm(*dev1, out_dtype=torch.float32, workspace=ws)
        o2 = B.nvfp4_gemm(*dev2, out_dtype=torch.float32, workspace=ws)
        U.assert_within(o1.cpu().numpy(), C1, T1, "product 1")
        U.assert_within(o2.cpu().numpy(), C2, T2, "product 2")


def test_m16_split_graph_replays():
    """The split kernel inside a replayed HIP graph: every replay equals the eager result (the
    counters return to zero, so nothing needs clearing between replays)."""
    M, K, N = 16, 25600, 1024
    dev, C, T = _pair(M, K, N, 9)
    ws = B.gemm_workspace(M, K, N, torch.device(U.DEV))
    assert ws is not None
    eager = B.nvfp4_gemm(*dev, out_dtype=torch.float32, workspace=ws).clone()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.nvfp4_gemm(*dev, out_dtype=torch.float32, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        B.nvfp4_gemm(*dev, out_dtype=torch.float32, out=out, workspace=ws)
    for _ in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32))
    U.assert_within(eager.cpu().numpy(), C, T, "graph")


def test_workspace_validation():
    lib = B.load()
    assert lib.nvfp4_gemm_workspace_bytes(2, 25600, 5120) == 0   # one or two rows: the GEMV
    assert lib.nvfp4_gemm_workspace_bytes(17, 25600, 5120) == 0  # tiled path
    assert lib.nvfp4_gemm_workspace_bytes(16, 25616, 5120) == 0  # K not a multiple of 128
    assert lib.nvfp4_gemm_workspace_bytes(16, 25600, 5120) > 0
    t = torch.zeros((8192,), dtype=torch.uint8, device=U.DEV)  # covers every operand if launched
    p = t.data_ptr()
    args = (16, 256, 16, p, p, p, p, p, p, p, B.NVFP4_F32)
    assert lib.nvfp4_gemm_ws(*args, p, -1, None) == B.NVFP4_ERR_SHAPE
    assert lib.nvfp4_gemm_ws(*args, None, 64, None) == B.NVFP4_ERR_NULL
    assert lib.nvfp4_gemm_ws(*args, p + 8, 32, None) == B.NVFP4_ERR_ALIGN
