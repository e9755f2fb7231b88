"""Pins for the oracle's NVFP4 GEMM (CPU only).

Exact rational brute force on tiny shapes, the blockwise (per-16-block partial
sum) form of the same product, one-hot and repeated-row closed forms.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q


def _quant(x):
    g = Q.global_scale(x)
    p, s = Q.quantize_packed(x, g)
    return p, s, g


def _exact_product(ap, asc, ga, wp, wsc, gw):
    """C as exact rationals: decode every element from its bits and sum without rounding."""
    e2m1 = {c: Fraction(float(v)) for c, v in enumerate(F.decode_e2m1(np.arange(16)))}
    e4m3 = {b: Fraction(float(v)) for b, v in enumerate(F.decode_e4m3(np.arange(0x7F)))}
    qa, qw = Q.unpack(ap), Q.unpack(wp)
    M, K = qa.shape
    N = qw.shape[0]
    ga, gw = Fraction(float(ga)), Fraction(float(gw))
    C = [[Fraction(0)] * N for _ in range(M)]
    for m, n, k in itertools.product(range(M), range(N), range(K)):
        a = e2m1[int(qa[m, k])] * e4m3[int(asc[m, k // 16])] * ga
        w = e2m1[int(qw[n, k])] * e4m3[int(wsc[n, k // 16])] * gw
        C[m][n] += a * w
    return C


@pytest.mark.parametrize("M,K,N", [(1, 16, 1), (2, 32, 3), (3, 64, 4), (4, 32, 8), (1, 48, 5)])
def test_gemm_matches_exact_rational_bruteforce(M, K, N):
    rng = np.random.default_rng(M * 100 + K + N)
    A = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    ap, asc, ga = _quant(A)
    wp, wsc, gw = _quant(W)
    C, T = G.gemm_ref(ap, asc, ga, wp, wsc, gw)
    exact = _exact_product(ap, asc, ga, wp, wsc, gw)
    for m in range(M):
        for n in range(N):
            ref = exact[m][n]
            assert abs(Fraction(C[m, n]) - ref) <= Fraction(1, 10 ** 12) * (abs(ref) + Fraction(T[m, n])), (m, n)
    Cb = G.gemm_blockwise(ap, asc, ga, wp, wsc, gw)
    np.testing.assert_allclose(Cb, C, rtol=1e-12, atol=1e-12 * np.max(T))


def test_tolerance_is_sum_of_abs_products():
    rng = np.random.default_rng(9)
    A = rng.standard_normal((2, 32)).astype(np.float32)
    W = rng.standard_normal((3, 32)).astype(np.float32)
    ap, asc, ga = _quant(A)
    wp, wsc, gw = _quant(W)
    C, T = G.gemm_ref(ap, asc, ga, wp, wsc, gw)
    exact_abs = [[sum(abs(x) for x in row) for row in pair] for pair in
                 [[[a * w for a, w in zip(ar, wr)] for wr in Q.dequantize(wp, wsc, gw)]
                  for ar in Q.dequantize(ap, asc, ga)]]
    np.testing.assert_allclose(T, 1e-3 * np.array(exact_abs), rtol=1e-12)
    assert np.all(np.abs(C) <= T / 1e-3 * (1 + 1e-12))


def test_one_hot_row_returns_weight_column():
    rng = np.random.default_rng(10)
    K, N = 64, 7
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wp, wsc, gw = _quant(W)
    a = np.zeros((1, K), np.float32)
    a[0, 37] = 2.625
    ap, asc, ga = _quant(a)
    # a quantizes exactly: amax = 2688 * 2^-10 -> g = 2^-10, block scale 448, element 6 * 448 * g
    assert ga == 2.0 ** -10 and Q.dequantize(ap, asc, ga)[0, 37] == 2.625
    C, _ = G.gemm_ref(ap, asc, ga, wp, wsc, gw)
    np.testing.assert_array_equal(C[0], 2.625 * Q.dequantize(wp, wsc, gw)[:, 37])


def test_identical_rows_identical_outputs_and_chunking():
    rng = np.random.default_rng(12)
    A = np.repeat(rng.standard_normal((1, 256)).astype(np.float32), 3, axis=0)
    W = (rng.standard_normal((40, 256)) * 0.02).astype(np.float32)
    ap, asc, ga = _quant(A)
    wp, wsc, gw = _quant(W)
    C1, _ = G.gemm_ref(ap, asc, ga, wp, wsc, gw, n_chunk=7)
    C2, _ = G.gemm_ref(ap, asc, ga, wp, wsc, gw, n_chunk=4096)
    assert np.array_equal(C1[0], C1[1]) and np.array_equal(C1[0], C1[2])
    np.testing.assert_allclose(C1, C2, rtol=1e-13)


def test_argmax_ties_go_low():
    C = np.array([[1.0, 3.0, 3.0], [2.0, 2.0, 2.0]])
    assert G.argmax_rows(C).tolist() == [1, 0]


def test_within_tolerance_mask():
    ref = np.array([1.0, 2.0])
    tol = np.array([0.1, 0.1])
    assert G.within_tolerance(np.array([1.05, 2.2], np.float32), ref, tol).tolist() == [True, False]
