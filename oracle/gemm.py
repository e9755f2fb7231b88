"""Oracle: NVFP4 W4A4 GEMM reference and its error bound (test infrastructure).

What the GEMM computes is the plain definition: with A and W dequantized
(x_hat = E2M1(code) * E4M3(scale) * g, see oracle.quant),

    C[m, n] = sum_k  a_hat[m, k] * w_hat[n, k]

accumulated in float64.  This is the matrix product of every linear layer of
the NVFP4 W4A4 model on the page "TensorRT Edge-LLM Completes the MLPerf Edge
Agentic Benchmark 6.4x Faster on Jetson AGX Thor" (section "Using NVFP4
quantization to accelerate Qwen3.6-27B inference": weights and activations in
NVFP4, LM head included).  W is stored [N, K] (K contiguous), so C = A_hat @ W_hat^T.

A GPU result is accepted when |gpu - C| <= 1e-3 * sum_k |a_hat[m,k] * w_hat[n,k]|
for every output element; `tolerance` returns that bound.
"""
from __future__ import annotations

import numpy as np

from .quant import BLOCK, dequantize, unpack
from .formats import decode_e2m1, decode_e4m3

REL_TOL = 1e-3


def gemm_ref(a_packed, a_scales, g_a, w_packed, w_scales, g_w, *, n_chunk: int = 4096,
             want_tol: bool = True):
    """float64 C [M, N] (and the per-element tolerance) from packed NVFP4 operands.

    The weight matrix is dequantized `n_chunk` rows at a time to bound memory.
    """
    a_hat = dequantize(a_packed, a_scales, g_a)          # [M, K]
    a_abs = np.abs(a_hat)
    N = np.asarray(w_packed).shape[0]
    M = a_hat.shape[0]
    C = np.empty((M, N), dtype=np.float64)
    T = np.empty((M, N), dtype=np.float64) if want_tol else None
    for n0 in range(0, N, n_chunk):
        w_hat = dequantize(w_packed[n0:n0 + n_chunk], w_scales[n0:n0 + n_chunk], g_w)
        C[:, n0:n0 + n_chunk] = a_hat @ w_hat.T
        if want_tol:
            T[:, n0:n0 + n_chunk] = REL_TOL * (a_abs @ np.abs(w_hat).T)
    return (C, T) if want_tol else C


def gemm_blockwise(a_packed, a_scales, g_a, w_packed, w_scales, g_w):
    """The same product grouped by 16-blocks: g_a*g_w*sum_b s_a*s_w*sum_{k in b} qa*qw.

    Used only to cross-check gemm_ref on small shapes (the two agree to float64 rounding).
    """
    qa = decode_e2m1(unpack(a_packed))
    qw = decode_e2m1(unpack(w_packed))
    M, K = qa.shape
    N = qw.shape[0]
    nb = K // BLOCK
    sa = decode_e4m3(a_scales)
    sw = decode_e4m3(w_scales)
    part = np.einsum("mbi,nbi->mnb", qa.reshape(M, nb, BLOCK), qw.reshape(N, nb, BLOCK))
    return float(g_a) * float(g_w) * np.einsum("mnb,mb,nb->mn", part, sa, sw)


def within_tolerance(gpu, ref, tol) -> np.ndarray:
    """Boolean mask of outputs that satisfy |gpu - ref| <= tol (gpu widened to float64)."""
    return np.abs(np.asarray(gpu, dtype=np.float64) - ref) <= tol


def argmax_rows(C) -> np.ndarray:
    """Row-wise argmax; ties resolve to the lowest index (numpy's rule)."""
    return np.argmax(np.asarray(C), axis=1)
