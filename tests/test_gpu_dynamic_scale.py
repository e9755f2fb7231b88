"""GPU parity of the dynamic activation scale (nvfp4_act_global_scale): g_a = fl32(amax|A| / 2688)
computed on the device equals the oracle's global_scale bit for bit (amax is exact and the division
correctly rounded), on the one-workgroup path (up to 2^20 elements) and the atomic path beyond, and a
decode step quantized with it matches the oracle.  Page "TensorRT Edge-LLM Completes the MLPerf Edge
Agentic Benchmark 6.4x Faster on Jetson AGX Thor", section "Using NVFP4 quantization to accelerate
Qwen3.6-27B inference" (NVFP4 activations; the dynamic scale is the alternative to a calibrated one)."""
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


@pytest.mark.parametrize("M,K", [(1, 16), (1, 5120), (2, 5120), (16, 25600), (64, 16384), (512, 5120), (3, 1040)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_scale_matches_oracle(M, K, dtype):
    rng = np.random.default_rng(M + K)
    A = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-3, 3))).astype(np.float32)
    A.reshape(-1)[rng.integers(0, M * K)] *= 37.0  # one outlier sets the maximum
    if dtype == torch.bfloat16:
        bits = WL.f32_to_bf16_bits(A)
        a, A_seen = U.dev_bf16_bits(bits), WL.bf16_bits_to_f32(bits)
    else:
        a, A_seen = U.dev_f32(A), A
    g = B.nvfp4_act_global_scale(a)
    assert U.f32_bits(g.item()) == U.f32_bits(Q.global_scale(A_seen)), (M, K, g.item(), Q.global_scale(A_seen))


def test_zero_activations_give_zero_scale():
    for M, K in ((1, 4096), (700, 2048)):
        g = B.nvfp4_act_global_scale(torch.zeros((M, K), dtype=torch.bfloat16, device="cuda"))
        assert g.item() == 0.0


def test_decode_step_with_dynamic_scale():
    """Decode up-projection (1 x 5120 x 25600, outlier channels) with g_a computed on the device:
    codes equal the oracle's quantization with the same formula; sampled outputs within the bar."""
    wl = WL.get("decode_up")
    inp = WL.generate(wl)
    A_seen = inp.a_f32()
    a = U.dev_acts(inp)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(inp.W))
    ga = B.nvfp4_act_global_scale(a)
    out, ac, asc = B.nvfp4_quantize_gemm(a, ga, wc, ws, gw)
    torch.cuda.synchronize()
    g_a = Q.global_scale(A_seen)
    assert U.f32_bits(ga.item()) == U.f32_bits(g_a)
    ap, asp = Q.quantize_packed(A_seen, g_a)
    np.testing.assert_array_equal(U.host(ac), ap)
    np.testing.assert_array_equal(U.host(asc), asp)
    cols = np.random.default_rng(5).choice(wl.N, size=128, replace=False)
    g_w = Q.global_scale(inp.W)
    wp, wsp = Q.quantize_packed(inp.W[cols], g_w)
    C, T = G.gemm_ref(ap, asp, g_a, wp, wsp, g_w)
    U.assert_within(U.host(out)[:, cols], C, T + U.out_rounding_slack(C, torch.bfloat16), "dynamic g_a decode")


# nvfp4_quantize_gemm_dynamic: one kernel for M <= 2 with K % 1024 == 0 in [1024, 8192] (every
# workgroup reduces the rows' largest magnitude itself), otherwise the scale kernel followed by
# nvfp4_quantize_gemm.  Cases: the fused kernel at decode size (bf16, with outlier channels) and
# with fp32 rows, two rows, the smallest and largest fused K, an all-zero row, and unfused shapes
# (K outside the set, three rows).
DYN_CASES = [(1, 5120, 25600, torch.bfloat16), (1, 5120, 3000, torch.float32), (2, 4096, 1000, torch.bfloat16),
             (1, 1024, 513, torch.float32), (2, 8192, 700, torch.bfloat16), (1, 2048, 300, "zeros"),
             (1, 2304, 500, torch.bfloat16), (3, 5120, 800, torch.float32)]


@pytest.mark.parametrize("M,K,N,kind", DYN_CASES, ids=lambda v: str(v).replace("torch.", ""))
def test_quantize_gemm_dynamic_matches_three_calls_and_oracle(M, K, N, kind):
    rng = np.random.default_rng(M * 7 + K + N)
    A = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-2, 2))).astype(np.float32)
    A[:, rng.choice(K, size=max(1, K // 200), replace=False)] *= 20.0  # outlier channels
    dtype = torch.bfloat16 if kind == "zeros" else kind
    if kind == "zeros":
        A[:] = 0.0
    if dtype == torch.bfloat16:
        bits = WL.f32_to_bf16_bits(A)
        a, A_seen = U.dev_bf16_bits(bits), WL.bf16_bits_to_f32(bits)
    else:
        a, A_seen = U.dev_f32(A), A
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(W))
    for out_dtype in (torch.bfloat16, torch.float32):
        out, ac, asc, ga = B.nvfp4_quantize_gemm_dynamic(a, wc, ws, gw, out_dtype=out_dtype)
        ga3 = B.nvfp4_act_global_scale(a)
        out3, ac3, asc3 = B.nvfp4_quantize_gemm(a, ga3, wc, ws, gw, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert U.f32_bits(ga.item()) == U.f32_bits(ga3.item())
        assert torch.equal(ac, ac3) and torch.equal(asc, asc3)
        assert torch.equal(out.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                           out3.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32))
    g_a = Q.global_scale(A_seen)
    assert U.f32_bits(ga.item()) == U.f32_bits(g_a)
    ap, asp = Q.quantize_packed(A_seen, g_a)
    np.testing.assert_array_equal(U.host(ac), ap)
    np.testing.assert_array_equal(U.host(asc), asp)
    cols = np.random.default_rng(3).choice(N, size=min(N, 96), replace=False)
    wp, wsp = Q.quantize_packed(W[cols], Q.global_scale(W))
    C, T = G.gemm_ref(ap, asp, g_a, wp, wsp, Q.global_scale(W))
    U.assert_within(U.host(out)[:, cols], C, T, f"M={M} K={K} N={N}")
