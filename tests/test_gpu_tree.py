"""GPU parity of greedy tree verification (nvfp4_tree_accept, nvfp4_tree_verify) against the oracle.

Page "TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x Faster on Jetson AGX
Thor", section "Using tree-based multi-token prediction to accelerate LLM inference": the target
verifies a 16-node candidate tree (8 draft steps, top-2 candidates per depth) in one LM-head pass at
temperature 0 and accepts the matching path.  Acceptance is integer work and must match the oracle
exactly.  At full size (the 16 x 5120 x 151936 LM head) every row's argmax must equal the oracle's
(its top-2 gaps are far above the fp32 accumulation error), and so must every greedy token and the
acceptance.  On the small random shapes the argmax of a row is decided in fp32 on the GPU; where
the oracle's exact logits put several columns within the error bound of the maximum, any of them
is a correct argmax, so the GPU's choice is checked against that admissible set (exactly where
the set is one column), and drafts never hinge on such a row: a child copies its parent's argmax
only where that argmax is unique, otherwise it carries a token outside the parent's admissible set.
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
from oracle import tree as TR

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    U.require_gpu_lib()


def i32(x) -> torch.Tensor:
    return torch.tensor(np.asarray(x, dtype=np.int32), device="cuda")


def tree16():
    """16 nodes over 8 depths: a main chain with one alternative sibling per depth 1..7 and a
    last node at depth 8."""
    parent, chain = [-1], [0]
    for _ in range(7):
        parent += [chain[-1], chain[-1]]
        chain.append(len(parent) - 2)
    parent.append(chain[-1])
    return parent


def expected_result(parent, draft, greedy):
    end, path, bonus = TR.accept(parent, draft, greedy)
    n = len(parent)
    return end, len(path), bonus, path + [-1] * (n - len(path))


def test_tree_accept_matches_oracle_on_random_trees():
    rng = np.random.default_rng(21)
    for trial in range(300):
        n = int(rng.integers(1, 17)) if trial % 10 else 64
        parent = [-1] + [int(rng.integers(0, v)) for v in range(1, n)]
        greedy = rng.integers(0, 4, size=n)
        draft = rng.integers(0, 4, size=n)
        for v in range(1, n):
            if rng.random() < 0.6:
                draft[v] = greedy[parent[v]]
        res = B.nvfp4_tree_accept(i32(parent), i32(draft), i32(greedy)).cpu().numpy().tolist()
        end, L, bonus, path = expected_result(parent, draft, greedy)
        assert res == [end, L, bonus] + path, (trial, parent, draft.tolist(), greedy.tolist())


def test_tree_accept_rejects_invalid_parents_without_faulting():
    # parent indices outside [0, v) reject the node (and its subtree)
    res = B.nvfp4_tree_accept(i32([-1, 0, 5, -7, 1]), i32([0, 3, 3, 3, 4]), i32([3, 4, 0, 0, 9])).cpu().tolist()
    assert res == [4, 2, 9, 1, 4, -1, -1, -1]


def make_drafts(rng, parent, adm, n_vocab):
    """Drafts from oracle information only: copy the parent's argmax where it is unique (with
    probability 0.75), else a token outside the parent's admissible set."""
    draft = [0]
    for v in range(1, len(parent)):
        a = adm[parent[v]]
        if len(a) == 1 and rng.random() < 0.75:
            draft.append(next(iter(a)))
        else:
            t = (max(a) + 1 + int(rng.integers(0, 1000))) % n_vocab
            while t in a:
                t = (t + 1) % n_vocab
            draft.append(t)
    return draft


def check_verify(ac, asc, ga, wc, wsc, gw, parent, draft, adm, greedy_ref, want_logits, C=None, T=None):
    greedy, result, logits = B.nvfp4_tree_verify(ac, asc, ga, wc, wsc, gw, i32(parent), i32(draft),
                                                 want_logits=want_logits)
    torch.cuda.synchronize()
    greedy = greedy.cpu().numpy()
    res = result.cpu().numpy().tolist()
    for v in range(len(parent)):
        assert int(greedy[v]) in adm[v], (v, int(greedy[v]), sorted(adm[v])[:8])
    end, L, bonus, path = expected_result(parent, draft, greedy_ref)
    assert res[0] == end and res[1] == L and res[3:] == path, (res, end, L, path)
    assert res[2] in adm[end] and res[2] == int(greedy[end])
    if want_logits:
        host = logits.cpu().numpy()
        assert np.array_equal(np.argmax(host, axis=1), greedy)
        if C is not None:
            U.assert_within(host, C, T, "tree_verify logits")


@pytest.mark.parametrize("M,K,N", [(1, 256, 1), (3, 1024, 37), (16, 256, 2000), (16, 5120, 3000),
                                   (16, 1040, 515), (5, 2048, 777)])
@pytest.mark.parametrize("want_logits", [False, True])
def test_tree_verify_small(M, K, N, want_logits):
    if K % 256 and not want_logits:
        pytest.skip("unfused shapes need the logits buffer (covered with want_logits)")
    rng = np.random.default_rng(M * 1000 + K + N)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = rng.standard_normal((M, K)).astype(np.float32)
    g_a = Q.global_scale(A)
    wc, wsc, gw = B.nvfp4_quantize_weights(U.dev_f32(W))
    ac, asc = B.nvfp4_quantize_act(U.dev_f32(A), U.scalar(g_a))
    ap, asp = Q.quantize_packed(A, g_a)
    wp, wsp = Q.quantize_packed(W, Q.global_scale(W))
    C, T = G.gemm_ref(ap, asp, g_a, wp, wsp, Q.global_scale(W))
    adm = TR.admissible_argmax(C, T)
    parent = tree16()[:M] if M <= 16 else None
    draft = make_drafts(rng, parent, adm, N)
    check_verify(ac, asc, U.scalar(g_a), wc, wsc, gw, parent, draft, adm, TR.greedy_tokens(C), want_logits, C, T)


def _golden_admissible():
    adm = {}
    for line in open(os.path.join(GOLDEN, "lm_head_admissible.txt")):
        if line.startswith("#") or not line.strip():
            continue
        row, cols = line.split(";")
        adm[int(row)] = {int(c) for c in cols.split()}
    return [adm[m] for m in range(len(adm))]


def _golden_argmax():
    out = []
    for line in open(os.path.join(GOLDEN, "lm_head_argmax.txt")):
        if line.startswith("#") or not line.strip():
            continue
        out.append(int(line.split(";")[1]))
    return out


def exact_drafts(rng, parent, greedy, n_vocab):
    """Drafts that copy the parent's exact argmax with probability 0.75, else another token."""
    draft = [0]
    for v in range(1, len(parent)):
        g = int(greedy[parent[v]])
        draft.append(g if rng.random() < 0.75 else (g + 1 + int(rng.integers(0, 1000))) % n_vocab)
    return draft


@pytest.mark.parametrize("want_logits", [False, True])
def test_tree_verify_lm_head_full_size(want_logits):
    """The LM head over a 16-node tree at full size (16 x 5120 x 151936), the argmax fused into
    the GEMM (or taken from the written logits): every greedy token equals the oracle's argmax
    from the oracle-written golden file, and the acceptance equals the oracle's exactly."""
    wl = WL.get("lm_head")
    inp = WL.generate(wl)
    a = inp.a_f32()
    g_a = Q.global_scale(a)
    wc, wsc, gw = B.nvfp4_quantize_weights(U.dev_f32(inp.W))
    ac, asc = B.nvfp4_quantize_act(U.dev_acts(inp), U.scalar(g_a))
    greedy_ref = _golden_argmax()
    parent = tree16()
    for seed in range(4):
        draft = exact_drafts(np.random.default_rng(seed), parent, greedy_ref, wl.N)
        greedy, result, logits = B.nvfp4_tree_verify(ac, asc, U.scalar(g_a), wc, wsc, gw, i32(parent), i32(draft),
                                                     want_logits=want_logits)
        torch.cuda.synchronize()
        assert greedy.cpu().numpy().tolist() == greedy_ref
        end, L, bonus, path = expected_result(parent, draft, greedy_ref)
        assert result.cpu().numpy().tolist() == [end, L, bonus] + path, (seed, draft)
        if want_logits:
            assert np.array_equal(np.argmax(logits.cpu().numpy(), axis=1), np.asarray(greedy_ref))


def _stream_head(M, seed, K=5120, N=70000):
    """Random NVFP4 operands of an M x K x N head (default 5120 x 70000): random activation codes
    and scale bytes, random weight codes and moderate E4M3 scale bytes (2^-2 .. 2^1.875), drawn
    on the device from a seeded generator."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    rnd = lambda lo, hi, shape: torch.randint(lo, hi, shape, dtype=torch.uint8, device="cuda", generator=gen)
    ac, asc = rnd(0, 256, (M, K // 2)), rnd(0x28, 0x48, (M, K // 16))
    wc, wsc = rnd(0, 256, (N, K // 2)), rnd(0x28, 0x48, (N, K // 16))
    return ac, asc, U.scalar(np.float32(0.03)), wc, wsc, U.scalar(np.float32(0.0173))


@pytest.mark.parametrize("M,N", [(3, 70000), (9, 70000), (16, 70000), (11, 70003)])
def test_tree_verify_fused_acceptance_on_weight_stream(M, N):
    """At M x 5120 x N (N = 70000, or 70003 with a ragged last group of rows) the LM head runs on
    the persistent weight-stream kernel, whose last workgroup to finish folds the argmax keys and
    runs the acceptance in the same launch.  On random trees, the result equals the oracle's walk
    over the greedy tokens the call returns (themselves the argmax of the logits the same kernel
    writes), every call returns the same greedy tokens, and the key workspace (arrival counter
    included) is zero after every call."""
    ops = _stream_head(M, 40 + M, 5120, N)
    assert B.gemm_dispatch(M, 5120, N, 0) == B.KERNEL_M16_STREAM
    keys = torch.zeros(1024, dtype=torch.int64, device="cuda")
    g0, _, logits = B.nvfp4_tree_verify(*ops, i32([-1] + [0] * (M - 1)), i32([0] * M), want_logits=True, keys=keys)
    g0 = g0.cpu().numpy()
    assert np.array_equal(np.argmax(logits.cpu().numpy(), axis=1), g0)
    assert int(keys.abs().sum()) == 0
    rng = np.random.default_rng(M)
    for trial in range(8):
        parent = [-1] + [int(rng.integers(0, v)) for v in range(1, M)]
        draft = [0] + [int(g0[parent[v]]) if rng.random() < 0.7 else int(g0[parent[v]] + 1) % N
                       for v in range(1, M)]
        greedy, result, _ = B.nvfp4_tree_verify(*ops, i32(parent), i32(draft), want_logits=bool(trial % 2),
                                                keys=keys)
        torch.cuda.synchronize()
        assert greedy.cpu().numpy().tolist() == g0.tolist(), trial
        end, L, bonus, path = expected_result(parent, draft, g0)
        assert result.cpu().numpy().tolist() == [end, L, bonus] + path, (trial, parent, draft)
        assert int(keys.abs().sum()) == 0, trial


def test_tree_verify_fused_acceptance_rejects_invalid_parents():
    """The weight-stream kernel's fused walk: parent indices outside [0, v) reject the node
    even when its draft matches (the walk reads nothing outside the arrays)."""
    ops = _stream_head(5, 77)
    keys = torch.zeros(1024, dtype=torch.int64, device="cuda")
    g, _, _ = B.nvfp4_tree_verify(*ops, i32([-1, 0, 1, 2, 3]), i32([0] * 5), keys=keys)
    g = g.cpu().numpy().tolist()
    parent = [-1, 0, 5, -7, 1]
    draft = [0, g[0], g[0], g[0], g[1]]
    greedy, result, _ = B.nvfp4_tree_verify(*ops, i32(parent), i32(draft), keys=keys)
    assert greedy.cpu().numpy().tolist() == g
    assert result.cpu().numpy().tolist() == [4, 2, g[4], 1, 4, -1, -1, -1]
    assert int(keys.abs().sum()) == 0


def test_tree_verify_fused_acceptance_with_more_workgroups_than_cus():
    """16 x 1024 x 300000: 18750 groups of 16 rows, so the stream kernel's grid exceeds the CU
    count and some workgroups start only after others have finished; the last to take its ticket
    still sees every key.  Greedy tokens equal the argmax of the logits the same launch writes,
    the result equals the oracle's walk over them, and the key workspace is zero afterwards."""
    M, K, N = 16, 1024, 300000
    assert B.gemm_dispatch(M, K, N, 0) == B.KERNEL_M16_STREAM
    ops = _stream_head(M, 91, K, N)
    keys = torch.zeros(1024, dtype=torch.int64, device="cuda")
    g0, _, logits = B.nvfp4_tree_verify(*ops, i32([-1] + [0] * (M - 1)), i32([0] * M), want_logits=True, keys=keys)
    g0 = g0.cpu().numpy()
    assert np.array_equal(np.argmax(logits.cpu().numpy(), axis=1), g0)
    del logits
    parent = tree16()
    draft = [0] + [int(g0[parent[v]]) if v % 3 else int(g0[parent[v]] + 1) % N for v in range(1, M)]
    for rep in range(3):
        greedy, result, _ = B.nvfp4_tree_verify(*ops, i32(parent), i32(draft), keys=keys)
        torch.cuda.synchronize()
        assert greedy.cpu().numpy().tolist() == g0.tolist(), rep
        end, L, bonus, path = expected_result(parent, draft, g0)
        assert result.cpu().numpy().tolist() == [end, L, bonus] + path, rep
        assert int(keys.abs().sum()) == 0, rep
