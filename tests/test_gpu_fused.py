"""GPU parity of nvfp4_quantize_gemm (activation quantization fused into the GEMV).

The fused call must return exactly what nvfp4_quantize_act followed by nvfp4_gemm returns (the
same kernels' arithmetic), its activation codes and scales must equal the oracle's quantization
of the same raw rows bit for bit, and the product must meet the GEMM bar against the oracle:
|gpu - C| <= 1e-3 * sum_k |a_hat * w_hat|.  Shapes cover the single-kernel case (M <= 2, K a
multiple of 1024 up to 8192), the two-launch fallback (other M or K), ragged N, and the decode
up-projection at full size (page "TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark
6.4x Faster on Jetson AGX Thor", section on NVFP4 quantization: low-batch decode is bound by
memory traffic, which NVFP4 activations reduce).
"""
import numpy as np
import pytest
import torch

import gpu_util as U
from nvfp4_w4a4_block_amd import binding as B
from nvfp4_w4a4_block_amd import workloads as WL
from oracle import gemm as G
from oracle import quant as Q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    U.require_gpu_lib()


def _raw(A: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Device copy of A in dtype; bf16 inputs are rounded on the host so both sides see the
    same values."""
    t = torch.from_numpy(A)
    if dtype == torch.bfloat16:
        t = t.to(torch.bfloat16)
    return t.contiguous().to("cuda")


def _check(M, K, N, dtype, seed, out_dtype=torch.bfloat16):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = rng.standard_normal((M, K)).astype(np.float32)
    a = _raw(A, dtype)
    A_seen = a.float().cpu().numpy()            # the values the GPU quantizes
    g_a = Q.global_scale(A_seen)
    ga = U.scalar(g_a)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(W))
    out, ac, asc = B.nvfp4_quantize_gemm(a, ga, wc, ws, gw, out_dtype=out_dtype)
    # the two-call form on the same inputs
    ac2, asc2 = B.nvfp4_quantize_act(a, ga)
    out2 = B.nvfp4_gemm(ac2, asc2, ga, wc, ws, gw, out_dtype=out_dtype)
    torch.cuda.synchronize()
    what = f"M={M} K={K} N={N} {dtype} -> {out_dtype}"
    assert torch.equal(ac, ac2) and torch.equal(asc, asc2), what
    assert torch.equal(out.view(torch.int16) if out_dtype == torch.bfloat16 else out.view(torch.int32),
                       out2.view(torch.int16) if out_dtype == torch.bfloat16 else out2.view(torch.int32)), what
    # against the oracle
    ap, asp = Q.quantize_packed(A_seen, g_a)
    np.testing.assert_array_equal(U.host(ac), ap, err_msg=what)
    np.testing.assert_array_equal(U.host(asc), asp, err_msg=what)
    wp, wsp = Q.quantize_packed(W, Q.global_scale(W))
    C, T = G.gemm_ref(ap, asp, g_a, wp, wsp, Q.global_scale(W))
    U.assert_within(U.host(out), C, T + U.out_rounding_slack(C, out_dtype), what)


FUSED = [(1, 1024, 1), (1, 2048, 37), (2, 2048, 515), (1, 3072, 64), (2, 4096, 300),
         (1, 5120, 3000), (2, 5120, 2600), (1, 6144, 129), (1, 7168, 200), (1, 8192, 1500)]
FALLBACK = [(3, 5120, 64), (16, 1024, 40), (2, 8192, 100), (1, 1040, 33), (1, 256, 17)]


@pytest.mark.parametrize("M,K,N", FUSED + FALLBACK)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_gemm_matches_two_calls_and_oracle(M, K, N, dtype):
    _check(M, K, N, dtype, seed=M * 7919 + K + N, out_dtype=torch.float32 if N % 2 else torch.bfloat16)


def test_quantize_gemm_zero_activation_and_scale():
    """An all-zero row gives zero codes, zero scales and a zero product; g_a = 0 likewise."""
    K, N = 5120, 64
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(W))
    a = torch.zeros((1, K), dtype=torch.bfloat16, device="cuda")
    out, ac, asc = B.nvfp4_quantize_gemm(a, U.scalar(0.0), wc, ws, gw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(ac.abs().sum()) == 0 and int(asc.sum()) == 0
    assert float(out.abs().max()) == 0.0
    a = torch.ones((1, K), dtype=torch.bfloat16, device="cuda")
    out, ac, asc = B.nvfp4_quantize_gemm(a, U.scalar(0.0), wc, ws, gw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(asc.sum()) == 0 and float(out.abs().max()) == 0.0


def test_quantize_gemm_decode_full_size():
    """The decode up-projection (1 x 5120 x 25600, bf16 activations with outlier channels) at full
    size: identical to the two-call form, codes equal to the oracle's, sampled outputs within the
    bar (the oracle computes the sampled weight rows one by one)."""
    wl = WL.get("decode_up")
    inp = WL.generate(wl)
    A_seen = inp.a_f32()
    g_a = Q.global_scale(A_seen)
    ga = U.scalar(g_a)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(inp.W))
    a = U.dev_acts(inp)
    out, ac, asc = B.nvfp4_quantize_gemm(a, ga, wc, ws, gw)
    ac2, asc2 = B.nvfp4_quantize_act(a, ga)
    out2 = B.nvfp4_gemm(ac2, asc2, ga, wc, ws, gw)
    torch.cuda.synchronize()
    assert torch.equal(ac, ac2) and torch.equal(asc, asc2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    ap, asp = Q.quantize_packed(A_seen, g_a)
    np.testing.assert_array_equal(U.host(ac), ap)
    np.testing.assert_array_equal(U.host(asc), asp)
    cols = np.random.default_rng(11).choice(wl.N, size=256, replace=False)
    g_w = Q.global_scale(inp.W)
    wp, wsp = Q.quantize_packed(inp.W[cols], g_w)
    C, T = G.gemm_ref(ap, asp, g_a, wp, wsp, g_w)
    got = U.host(out)[:, cols]
    U.assert_within(got, C, T + U.out_rounding_slack(C, torch.bfloat16), "decode_up fused")
