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


# (M, K, N): one line (K = 128), odd line counts, 49 and 50 lines, K beyond the whole-range scale
# staging (64 lines: the 8-line scale blocks), N of 1, ragged and several row blocks.
CASES = [(3, 128, 1), (5, 384, 37), (16, 1024, 300), (7, 2688, 129), (16, 6272, 64), (16, 6400, 100),
         (16, 9216, 1000), (11, 25600, 300), (16, 5120, 3000), (4, 640, 2049), (1, 3456, 333), (2, 8320, 129)]


@pytest.mark.parametrize("M,K,N", CASES)
def test_m16_with_and_without_workspace(M, K, N):
    """The library's dispatch without and with a workspace (short-K products with N <= 16384 run
    the skinny kernel, long ones the M-tile kernel, split over workgroups when the workspace is
    there), and the M-tile kernel itself for every shape, unsplit."""
    dev, C, T = _pair(M, K, N, 11 * M + K + N)
    for i, ws in enumerate((None, "auto")):
        out_dtype = torch.float32 if i == 0 else torch.bfloat16
        out = B.nvfp4_gemm(*dev, out_dtype=out_dtype, workspace=ws)
        U.assert_within(U.host(out), C, T + U.out_rounding_slack(C, out_dtype), f"M={M} K={K} N={N} ws={ws}")
    out = B.nvfp4_gemm(*dev, out_dtype=torch.float32, path=B.KERNEL_M16)
    U.assert_within(U.host(out), C, T, f"M={M} K={K} N={N} M-tile kernel")


# Split shapes: the workspace plan splits K until there are about 7.5 waves per CU (at least 6
# lines per split): few rows and a long K give many splits, a larger N fewer.
SPLIT_CASES = [(16, 25600, 512), (16, 25600, 5120), (9, 12288, 333), (16, 10240, 2000), (3, 9216, 129)]


@pytest.mark.parametrize("M,K,N", SPLIT_CASES)
def test_m16_split_matches_oracle(M, K, N):
    need = int(B.load().nvfp4_gemm_workspace_bytes(M, K, N))
    assert need > 0, "the product should split"
    assert B.gemm_dispatch(M, K, N, need) == B.KERNEL_M16
    dev, C, T = _pair(M, K, N, 3 * M + K + N)
    ws = torch.zeros((need,), dtype=torch.uint8, device=U.DEV)
    for out_dtype in (torch.float32, torch.bfloat16):
        out = B.nvfp4_gemm(*dev, out_dtype=out_dtype, workspace=ws)
        U.assert_within(U.host(out), C, T + U.out_rounding_slack(C, out_dtype), f"M={M} K={K} N={N} split")
    assert not ws[:256].any().item(), "arrival counters not reset"


def test_m16_split_deterministic_and_counters_reset():
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


def test_m16_split_reads_fresh_partials():
    """Two different products through one workspace, alternately: every result must match its
    own oracle, so the last workgroup of a row block never adds partial sums left over from the
    other product (or from an earlier call) instead of the ones just written."""
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


def _replays_match(call, out, eager):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        call()
    for _ in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32))


def test_m16_split_graph_replays():
    """The split kernel inside a replayed HIP graph: every replay equals the eager result (the
    counters return to zero, so nothing needs clearing between replays)."""
    M, K, N = 16, 25600, 1024
    dev, C, T = _pair(M, K, N, 9)
    ws = B.gemm_workspace(M, K, N, torch.device(U.DEV))
    assert ws is not None
    eager = B.nvfp4_gemm(*dev, out_dtype=torch.float32, workspace=ws).clone()
    out = torch.empty_like(eager)
    _replays_match(lambda: B.nvfp4_gemm(*dev, out_dtype=torch.float32, out=out, workspace=ws), out, eager)
    U.assert_within(eager.cpu().numpy(), C, T, "graph")


def test_m16_unsplit_graph_replays():
    """The unsplit M-tile kernel (a product with enough rows to fill the GPU: no split even with
    a workspace) inside a replayed HIP graph."""
    M, K, N = 16, 5120, 20000
    assert B.gemm_dispatch(M, K, N, 1 << 24) == B.KERNEL_M16
    assert int(B.load().nvfp4_gemm_workspace_bytes(M, K, N)) == 0
    dev, C, T = _pair(M, K, N, 10)
    eager = B.nvfp4_gemm(*dev, out_dtype=torch.float32).clone()
    out = torch.empty_like(eager)
    _replays_match(lambda: B.nvfp4_gemm(*dev, out_dtype=torch.float32, out=out), out, eager)
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
