"""GPU parity of the NVFP4 W4A4 GEMV/GEMM against the CPU oracle.

Bar: |gpu - C| <= 1e-3 * sum_k |a_hat[m,k] * w_hat[n,k]| per output, C the fp64 product of the
oracle-dequantized operands.  Small shapes (several tiles, ragged tails, every path) compare
every output; the full-size workloads, in the launch configuration the benchmark uses, compare
sampled output columns (the oracle computes them one weight row at a time).  Shapes stand in
for the decode (M=1), 16-node tree verification (M=16) and suffix prefill (M=512) passes of
the page "TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x Faster on Jetson
AGX Thor" (sections on NVFP4 quantization, tree-based multi-token prediction and KV reuse).
"""
import os

import numpy as np
import pytest
import torch

import gpu_util as U
from nvfp4_w4a4_block_amd import binding as B
from nvfp4_w4a4_block_amd import workloads as WL
from oracle import gemm as G
from oracle import quant as Q

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    U.require_gpu_lib()


def _quantized_pair(A: np.ndarray, W: np.ndarray):
    """GPU quantization of both operands (bit-exactness is covered by test_gpu_quant) plus the
    oracle's own quantization of the same seeded inputs."""
    g_a = Q.global_scale(A)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(W))
    ac, asc = B.nvfp4_quantize_act(U.dev_f32(A), U.scalar(g_a))
    ref = (Q.quantize_packed(A, g_a), g_a, Q.quantize_packed(W, Q.global_scale(W)), Q.global_scale(W))
    return (ac, asc, U.scalar(g_a), wc, ws, gw), ref


def _oracle(ref, cols=None):
    (ap, asc), g_a, (wp, wsc), g_w = ref
    if cols is not None:
        wp, wsc = wp[cols], wsc[cols]
    return G.gemm_ref(ap, asc, g_a, wp, wsc, g_w)


MS = [1, 2, 5, 15, 16, 17, 33, 64, 127, 128, 129, 256]
KNS = [(16, 1), (32, 17), (48, 40), (256, 256), (1040, 300), (4096, 160)]
PATHS = [B.PATH_AUTO, B.PATH_SKINNY, B.PATH_TILED]


@pytest.mark.parametrize("K,N", KNS)
@pytest.mark.parametrize("M", MS)
def test_gemm_small_shapes_all_paths(M, K, N):
    rng = np.random.default_rng(1000 * M + K + N)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = rng.standard_normal((M, K)).astype(np.float32)
    dev, ref = _quantized_pair(A, W)
    C, T = _oracle(ref)
    for i, path in enumerate(PATHS):
        out_dtype = torch.bfloat16 if (i + M) % 2 else torch.float32
        out = B.nvfp4_gemm(*dev, out_dtype=out_dtype, path=path)
        U.assert_within(U.host(out), C, T + U.out_rounding_slack(C, out_dtype),
                        f"M={M} K={K} N={N} path={path} {out_dtype}")


# The persistent tiled kernel (K % 1024 == 0, M > 16): 64 x 160 tiles, 256-K steps, scale bytes
# fetched four steps at a time, loads three steps ahead across tile boundaries.  Cases: one scale
# group, ragged M and N, more tiles than workgroups (600 and 262 tiles: several tiles per
# workgroup, with and without a tile count divisible by 8), a single tile, M just above 16.  K %
# 256 == 0 shapes outside that rule (768, 1280) take the simple tiled kernel.
TILED_CASES = [(129, 1024, 300), (200, 2048, 1000), (300, 3072, 16000), (129, 1024, 10480), (512, 4096, 80),
               (17, 1024, 2000), (129, 768, 300), (200, 1280, 1000)]


@pytest.mark.parametrize("M,K,N", TILED_CASES)
def test_gemm_tiled_persistent(M, K, N):
    rng = np.random.default_rng(7 * M + K + N)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = rng.standard_normal((M, K)).astype(np.float32)
    dev, ref = _quantized_pair(A, W)
    C, T = _oracle(ref)
    for out_dtype in (torch.float32, torch.bfloat16):
        out = B.nvfp4_gemm(*dev, out_dtype=out_dtype, path=B.PATH_TILED)
        U.assert_within(U.host(out), C, T + U.out_rounding_slack(C, out_dtype), f"M={M} K={K} N={N} {out_dtype}")


# One or two activation rows with K >= 2048 and K % 256 == 0 take the memory-order GEMV: rows
# whose chunk count (K/32) is not a multiple of 64, row runs that wrap inside an instruction,
# several rows per wave (N above the resident wave count), a single row; K = 2080 (odd chunk
# count, scale rows not 16-byte aligned) is served by the general kernel.
GEMV_KNS = [(2048, 1), (2080, 64), (2080, 37), (3072, 515), (2304, 3000), (5120, 2600)]


@pytest.mark.parametrize("K,N", GEMV_KNS)
@pytest.mark.parametrize("M", [1, 2])
def test_gemv_ragged_shapes(M, K, N):
    rng = np.random.default_rng(7 * M + K + 3 * N)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = rng.standard_normal((M, K)).astype(np.float32)
    dev, ref = _quantized_pair(A, W)
    C, T = _oracle(ref)
    for out_dtype in (torch.float32, torch.bfloat16):
        out = B.nvfp4_gemm(*dev, out_dtype=out_dtype)
        U.assert_within(U.host(out), C, T + U.out_rounding_slack(C, out_dtype), f"M={M} K={K} N={N} {out_dtype}")


def test_gemm_deterministic_and_paths_agree_at_m16():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((1000, 5120)) * 0.02).astype(np.float32)
    A = rng.standard_normal((16, 5120)).astype(np.float32)
    dev, ref = _quantized_pair(A, W)
    C, T = _oracle(ref)
    outs = {}
    for path in (B.PATH_SKINNY, B.PATH_TILED):
        o1 = B.nvfp4_gemm(*dev, out_dtype=torch.float32, path=path).cpu().numpy()
        o2 = B.nvfp4_gemm(*dev, out_dtype=torch.float32, path=path).cpu().numpy()
        assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32)), f"path {path} not deterministic"
        U.assert_within(o1, C, T, f"path {path}")
        outs[path] = o1
    assert np.all(np.abs(outs[B.PATH_SKINNY].astype(np.float64) - outs[B.PATH_TILED]) <= 2 * T)


def test_gemm_zero_operands():
    """A zero activation tensor (g_a = 0) gives exact zeros, and so do zero weights."""
    rng = np.random.default_rng(8)
    W = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    for A, Wm in ((np.zeros((3, 256), np.float32), W), (rng.standard_normal((3, 256)).astype(np.float32),
                                                        np.zeros_like(W))):
        dev, _ = _quantized_pair(A, Wm)
        for path in PATHS:
            assert not B.nvfp4_gemm(*dev, out_dtype=torch.float32, path=path).any().item()


def test_gemm_empty():
    e = torch.empty((0, 16), dtype=torch.uint8, device=U.DEV)
    s = torch.empty((0, 2), dtype=torch.uint8, device=U.DEV)
    g = U.scalar(np.float32(1))
    w = torch.zeros((5, 16), dtype=torch.uint8, device=U.DEV)
    ws = torch.zeros((5, 2), dtype=torch.uint8, device=U.DEV)
    assert B.nvfp4_gemm(e, s, g, w, ws, g).shape == (0, 5)
    assert B.nvfp4_gemm(w, ws, g, e, s, g).shape == (5, 0)


# ---------------------------------------------------------------------------
# Full-size workloads, auto path (the launch configuration the benchmark times).
# ---------------------------------------------------------------------------

_FULL_ORACLE: dict = {}


def full_oracle(name):
    """The oracle's product of a whole workload (every output), from the seeded inputs; cached
    for the module (the weight quantization is ~15 s per 131M-element matrix)."""
    if name not in _FULL_ORACLE:
        wl = WL.get(name)
        inp = WL.generate(wl)
        a = inp.a_f32()
        g_a = Q.global_scale(a)
        g_w = Q.global_scale(inp.W)
        ap, asp = Q.quantize_packed(a, g_a)
        C = np.empty((wl.M, wl.N))
        T = np.empty((wl.M, wl.N))
        for n0 in range(0, wl.N, 4096):
            wp, wsp = Q.quantize_packed(inp.W[n0:n0 + 4096], g_w)
            C[:, n0:n0 + 4096], T[:, n0:n0 + 4096] = G.gemm_ref(ap, asp, g_a, wp, wsp, g_w)
        _FULL_ORACLE[name] = (wl, inp, g_a, C, T)
    return _FULL_ORACLE[name]


def stored_bound(C, T, out_dtype):
    """The bound for a stored result: the GEMM tolerance, plus for a bf16 result the rounding of
    the fp32 value v (|v - C| <= T) to bf16, at most half an ulp: 2^-8 |v| <= 2^-8 (|C| + T)."""
    if out_dtype == torch.bfloat16:
        return T + 2.0 ** -8 * (np.abs(C) + T)
    return T


@pytest.mark.parametrize("name,workspace", [("decode_up", "auto"), ("verify_down", "auto"), ("verify_down", None)])
def test_full_size_every_output(name, workspace):
    """Every output of the decode up-projection (1 x 5120 x 25600, FP4 GEMV) and of the tree-
    verification down-projection (16 x 25600 x 5120, split M-tile kernel with the workspace, the
    skinny kernel without), in the benchmark's launch configuration."""
    wl, inp, g_a, C, T = full_oracle(name)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(inp.W))
    ac, asc = B.nvfp4_quantize_act(U.dev_acts(inp), U.scalar(g_a))
    out_dtype = torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32
    out = U.host(B.nvfp4_gemm(ac, asc, U.scalar(g_a), wc, ws, gw, out_dtype=out_dtype, workspace=workspace))
    print(f"{name}: {int(np.sum(np.abs(out - C) > T))} of {C.size} outputs need the bf16 rounding allowance")
    U.assert_within(out, C, stored_bound(C, T, out_dtype), f"{name} workspace={workspace}")


def test_full_size_decode_fused_every_output():
    """The decode step as the benchmark runs it: nvfp4_quantize_gemm (activation quantization
    inside the FP4 GEMV, one kernel) on the raw bf16 row; every output, and the activation codes
    and scales bit-exact."""
    wl, inp, g_a, C, T = full_oracle("decode_up")
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(inp.W))
    out, ac, asc = B.nvfp4_quantize_gemm(U.dev_acts(inp), U.scalar(g_a), wc, ws, gw, out_dtype=torch.bfloat16)
    ap, asp = Q.quantize_packed(inp.a_f32(), g_a)
    assert np.array_equal(ac.cpu().numpy(), ap) and np.array_equal(asc.cpu().numpy(), asp)
    U.assert_within(U.host(out), C, stored_bound(C, T, torch.bfloat16), "decode_up fused")


def _sampled(name, n_sample=384):
    wl = WL.get(name)
    inp = WL.generate(wl)
    a = inp.a_f32()
    g_a = Q.global_scale(a)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(inp.W))
    ac, asc = B.nvfp4_quantize_act(U.dev_acts(inp), U.scalar(g_a))
    out_dtype = torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32
    out = U.host(B.nvfp4_gemm(ac, asc, U.scalar(g_a), wc, ws, gw, out_dtype=out_dtype, workspace="auto"))
    rng = np.random.default_rng(3)
    cols = np.unique(np.concatenate([[0, wl.N - 1], rng.choice(wl.N, min(n_sample, wl.N), replace=False)]))
    g_w = Q.global_scale(inp.W)
    ap, asp = Q.quantize_packed(a, g_a)
    wp, wsp = Q.quantize_packed(inp.W[cols], g_w)
    C, T = G.gemm_ref(ap, asp, g_a, wp, wsp, g_w)
    return wl, out, cols, C, T


@pytest.mark.parametrize("name", ["tiny", "lm_head"])
def test_full_size_sampled_outputs(name):
    """The tiny GEMV (every output: 256 columns) and sampled columns of the 151936-column LM head
    (the oracle would need ~3 minutes for all of them; its argmax is checked exactly below)."""
    wl, out, cols, C, T = _sampled(name)
    assert wl.out_dtype == "f32"
    U.assert_within(out[:, cols], C, T, name)


def _golden_lm_head():
    rows = []
    with open(os.path.join(GOLDEN, "lm_head_argmax.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            m, best, vbest, second, vsecond, tol = [t.strip() for t in line.split(";")]
            rows.append((int(m), int(best), float(vbest), int(second), float(vsecond), float(tol)))
    return rows


def _golden_admissible():
    adm = {}
    for line in open(os.path.join(GOLDEN, "lm_head_admissible.txt")):
        if line.startswith("#") or not line.strip():
            continue
        row, cols = line.split(";")
        adm[int(row)] = {int(c) for c in cols.split()}
    return [adm[m] for m in range(len(adm))]


def fp32_accumulation_estimate(K: int, tol: float) -> float:
    """Typical error of an fp32 sum of K exact products whose magnitudes add up to
    S = tol / 1e-3: rounding errors of random sign, u * sqrt(K) * S with u = 2^-24."""
    return 2.0 ** -24 * np.sqrt(K) * tol / G.REL_TOL


def test_lm_head_argmax_matches_oracle():
    """Per-row argmax of the full 151936-column NVFP4 LM head equals the oracle's exactly, on all
    16 rows (the tree acceptance at temperature 0 compares argmax tokens).  The golden margins
    make this well posed: every row's top-2 gap is more than 40 times the typical fp32
    accumulation error of the two logits, and the GPU logits at both columns are measured to be
    well inside half the gap."""
    wl = WL.get("lm_head")
    inp = WL.generate(wl)
    a = inp.a_f32()
    g_a = Q.global_scale(a)
    wc, ws, gw = B.nvfp4_quantize_weights(U.dev_f32(inp.W))
    ac, asc = B.nvfp4_quantize_act(U.dev_acts(inp), U.scalar(g_a))
    logits = B.nvfp4_gemm(ac, asc, U.scalar(g_a), wc, ws, gw, out_dtype=torch.float32)
    top = torch.argmax(logits, dim=1).cpu().numpy()
    host = logits.cpu().numpy()
    gold = _golden_lm_head()
    adm = _golden_admissible()
    assert len(gold) == wl.M == len(adm)
    for m, best, vbest, second, vsecond, tol in gold:
        gap = vbest - vsecond
        est = fp32_accumulation_estimate(wl.K, tol)
        assert gap > 40 * 2 * est, (m, gap, est)  # the seed gives no near-tie
        err_b, err_s = abs(host[m, best] - vbest), abs(host[m, second] - vsecond)
        print(f"row {m}: argmax {best} gap {gap:.4g} fp32 estimate {est:.3g} measured errors "
              f"{err_b:.3g} {err_s:.3g} tol {tol:.3g} admissible set {sorted(adm[m])}")
        assert err_b + err_s < gap / 2, (m, err_b, err_s, gap)
        assert err_b <= tol
        assert int(top[m]) == best, (m, int(top[m]), best, float(host[m, top[m]]), vbest)


def test_prefill_chain_up_then_down():
    """Suffix prefill: up-projection (512 x 5120 -> 25600), re-quantization of its bf16 output
    with a static scale, down-projection (25600 -> 5120).  The oracle runs the whole chain from
    the seeded inputs on its own; the activation scale of the second GEMM is calibrated on the
    oracle's first-GEMM output for a sample of rows."""
    wl = WL.get("prefill")
    inp = WL.generate(wl)
    M, K, N = wl.M, wl.K, wl.N
    a = inp.a_f32()
    g1 = Q.global_scale(a)
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 14, replace=False)]))
    cols1 = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 126, replace=False)]))

    # oracle: GEMM1 on the sampled rows (all columns: needs all of W1) and on sampled columns,
    # GEMM2 on every column of the sampled rows
    gw1 = Q.global_scale(inp.W)
    gw2 = Q.global_scale(inp.W2)
    ap, asp = Q.quantize_packed(a, g1)
    w1p, w1s = Q.quantize_packed(inp.W, gw1)
    C1r, T1r = G.gemm_ref(ap[rows], asp[rows], g1, w1p, w1s, gw1)
    C1c, T1c = G.gemm_ref(ap, asp, g1, w1p[cols1], w1s[cols1], gw1)
    y1r_bits = WL.f32_to_bf16_bits(C1r.astype(np.float32))   # the oracle's bf16 Y1 (see below)
    y1r = WL.bf16_bits_to_f32(y1r_bits)
    g2 = Q.global_scale(y1r)
    a2p, a2s = Q.quantize_packed(y1r, g2)
    C2 = np.empty((len(rows), K))
    T2 = np.empty((len(rows), K))
    for k0 in range(0, K, 1024):
        w2p, w2s = Q.quantize_packed(inp.W2[k0:k0 + 1024], gw2)
        C2[:, k0:k0 + 1024], T2[:, k0:k0 + 1024] = G.gemm_ref(a2p, a2s, g2, w2p, w2s, gw2)

    # GPU chain, exactly as the benchmark runs it
    wc1, ws1, gw1_d = B.nvfp4_quantize_weights(U.dev_f32(inp.W))
    wc2, ws2, gw2_d = B.nvfp4_quantize_weights(U.dev_f32(inp.W2))
    ac1, as1 = B.nvfp4_quantize_act(U.dev_acts(inp), U.scalar(g1))
    y1, ac2, as2 = B.nvfp4_gemm_quantize_output(ac1, as1, U.scalar(g1), wc1, ws1, gw1_d, U.scalar(g2),
                                                out_dtype=torch.bfloat16)
    y2 = B.nvfp4_gemm(ac2, as2, U.scalar(g2), wc2, ws2, gw2_d, out_dtype=torch.bfloat16)
    # the fused re-quantization equals quantizing the stored Y1 in a separate launch
    qc, qs = B.nvfp4_quantize_act(y1, U.scalar(g2))
    assert torch.equal(qc, ac2) and torch.equal(qs, as2)

    y1h = U.host(y1)
    U.assert_within(y1h[rows], C1r, stored_bound(C1r, T1r, torch.bfloat16), "GEMM1 sampled rows")
    U.assert_within(y1h[:, cols1], C1c, stored_bound(C1c, T1c, torch.bfloat16), "GEMM1 sampled columns")
    # Re-quantization: a block's codes are compared where both sides fed it the same 16 bf16
    # values (the fp32-accumulated GPU Y1 and the fp64 oracle Y1 round to bf16 identically
    # almost everywhere); such blocks must match bit for bit, and mismatched inputs must be rare.
    y1g_bits = y1[torch.as_tensor(rows, device=y1.device)].view(torch.int16).cpu().numpy().view(np.uint16)
    same = (y1g_bits == y1r_bits).reshape(len(rows), N // 16, 16).all(axis=2)
    assert same.mean() > 0.99, same.mean()
    gc = ac2[torch.as_tensor(rows, device=y1.device)].cpu().numpy().reshape(len(rows), N // 16, 8)
    gs = as2[torch.as_tensor(rows, device=y1.device)].cpu().numpy()
    assert np.array_equal(gs[same], a2s[same])
    assert np.array_equal(gc[same], a2p.reshape(len(rows), N // 16, 8)[same])
    U.assert_within(U.host(y2)[rows], C2, stored_bound(C2, T2, torch.bfloat16), "GEMM2 sampled rows, every column")
