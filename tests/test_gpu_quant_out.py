"""GPU parity of nvfp4_gemm_quantize_output: an NVFP4 product whose output is also emitted in
NVFP4 (one layer of a suffix prefill feeding the next; page "TensorRT Edge-LLM Completes the
MLPerf Edge Agentic Benchmark 6.4x Faster on Jetson AGX Thor", sections "Reusing KV cache across
agent turns" and "Using NVFP4 quantization to accelerate Qwen3.6-27B inference").

Bars: the output equals nvfp4_gemm's bit for bit and is within 1e-3 * sum|a*w| of the oracle's
fp64 product; its codes and scales equal nvfp4_quantize_act applied to the stored output bit for
bit; and, for bf16 outputs, on every 16-block whose stored values equal the oracle's own
bf16-rounded product, they equal the oracle quantizer's codes and scales of that product.
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


# (M, K, N): fused epilogue (M > 16, K % 1024 == 0): one tile, ragged M and N (N = 400 ends
# inside a tile of 160 columns), several tiles per workgroup; fallbacks (two launches): the
# weight-streaming path (M <= 16), the simple tiled kernel (K % 1024 != 0), the GEMV (M = 1).
CASES = [(17, 1024, 160), (129, 2048, 400), (512, 1024, 5120), (200, 3072, 1008),
         (16, 1024, 320), (64, 768, 96), (1, 2048, 256)]


@pytest.mark.parametrize("M,K,N", CASES)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_gemm_quantize_output(M, K, N, out_dtype):
    rng = np.random.default_rng(3 * M + K + N)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = rng.standard_normal((M, K)).astype(np.float32)
    g_a = Q.global_scale(A)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(W))
    ac, asc = B.nvfp4_quantize_act(U.dev_f32(A), U.scalar(g_a))
    ap, asp = Q.quantize_packed(A, g_a)
    wp, wsp = Q.quantize_packed(W, Q.global_scale(W))
    C, T = G.gemm_ref(ap, asp, g_a, wp, wsp, Q.global_scale(W))
    ref_out = C.astype(np.float32)
    if out_dtype == torch.bfloat16:
        ref_out = WL.bf16_bits_to_f32(WL.f32_to_bf16_bits(ref_out))
    g_y = Q.global_scale(ref_out)  # static scale calibrated on the oracle's output
    gy = U.scalar(g_y)

    out, yc, ys = B.nvfp4_gemm_quantize_output(ac, asc, U.scalar(g_a), wc, ws, gw, gy, out_dtype=out_dtype)
    plain = B.nvfp4_gemm(ac, asc, U.scalar(g_a), wc, ws, gw, out_dtype=out_dtype)
    assert torch.equal(out.view(torch.uint8), plain.view(torch.uint8)), "output differs from nvfp4_gemm"
    host = U.host(out)
    U.assert_within(host, C, T + U.out_rounding_slack(C, out_dtype), f"M={M} K={K} N={N}")

    qc, qs = B.nvfp4_quantize_act(out, gy)
    assert torch.equal(yc, qc) and torch.equal(ys, qs), "fused output quantization differs"

    if out_dtype != torch.bfloat16:
        return  # fp32 outputs match the oracle's only within tolerance, never bit for bit
    # against the oracle quantizer, on blocks whose stored values equal the oracle's own
    oc, osc = Q.quantize_packed(ref_out, g_y)
    same = (host.view(np.uint32) == ref_out.view(np.uint32)).reshape(M, N // 16, 16).all(axis=2)
    assert same.mean() > 0.9, same.mean()
    assert np.array_equal(yc.cpu().numpy().reshape(M, N // 16, 8)[same], oc.reshape(M, N // 16, 8)[same])
    assert np.array_equal(ys.cpu().numpy()[same], osc[same])


def test_gemm_quantize_output_zero_scale():
    """g_y = 0: every scale byte 0 and every code a signed zero, as the quantizer defines."""
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((320, 1024)) * 0.02).astype(np.float32)
    A = rng.standard_normal((64, 1024)).astype(np.float32)
    g_a = Q.global_scale(A)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(W))
    ac, asc = B.nvfp4_quantize_act(U.dev_f32(A), U.scalar(g_a))
    out, yc, ys = B.nvfp4_gemm_quantize_output(ac, asc, U.scalar(g_a), wc, ws, gw, U.scalar(np.float32(0)))
    assert not ys.any().item()
    assert torch.equal(yc & 0x77, torch.zeros_like(yc))
    qc, qs = B.nvfp4_quantize_act(out, U.scalar(np.float32(0)))
    assert torch.equal(yc, qc) and torch.equal(ys, qs)
