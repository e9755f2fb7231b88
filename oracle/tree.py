"""Oracle: greedy verification of a candidate tree over the LM head (test infrastructure).

Page "TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x Faster on Jetson AGX Thor",
section "Using tree-based multi-token prediction to accelerate LLM inference": a draft model
proposes high-probability candidates organized as a tree (the benchmark's server uses a 16-node
verification tree built from 8 draft steps with the top-2 candidates per depth), the target model
verifies every candidate in one forward pass, and the runtime accepts the matching path, advancing
by several tokens when several candidates are accepted.  The benchmark runs at temperature 0 (the
measurement settings on the same pages), so the target's choice after a node is the argmax of that
node's logits: one LM-head row per tree node, M = 16 rows of the NVFP4 GEMM.

The pages give no algorithm; the reading taken here is the plainest one they support:

* nodes 0 .. n-1 in topological order; node 0 is the root (the last token already in the
  sequence), parent[0] = -1 and 0 <= parent[v] < v for v >= 1; draft[v] is node v's candidate
  token (draft[0] is unused);
* greedy[v] = argmax of logits row v (the target's next token after the path root .. v), ties to
  the lowest token index;
* node v is accepted iff v == 0, or parent[v] is accepted and draft[v] == greedy[parent[v]];
* the accepted path ends at the deepest accepted node (the lowest index among equally deep ones);
  the path's draft tokens are emitted, then the bonus token greedy[end], so one verification
  step advances by depth(end) + 1 tokens.

Pinned by tests/test_oracle_tree.py: hand-worked trees (tests/golden/tree_accept.txt), an
exhaustive root-path search, the linear chain (longest matching prefix) and degenerate trees.
"""
from __future__ import annotations

import numpy as np


def greedy_tokens(logits) -> np.ndarray:
    """Row-wise argmax of [M, N] logits; ties to the lowest index (temperature-0 choice)."""
    return np.argmax(np.asarray(logits), axis=1).astype(np.int64)


def depths(parent) -> np.ndarray:
    """Depth of every node (root 0); raises on a parent array that is not a topological tree."""
    parent = np.asarray(parent, dtype=np.int64)
    n = parent.shape[0]
    if n < 1 or parent[0] != -1:
        raise ValueError("node 0 must be the root (parent -1)")
    d = np.zeros(n, dtype=np.int64)
    for v in range(1, n):
        p = int(parent[v])
        if not 0 <= p < v:
            raise ValueError(f"parent[{v}] = {p} is not an earlier node")
        d[v] = d[p] + 1
    return d


def accept(parent, draft, greedy):
    """(end node, accepted path nodes root-child first, bonus token) for one verification step."""
    parent = np.asarray(parent, dtype=np.int64)
    draft = np.asarray(draft, dtype=np.int64)
    greedy = np.asarray(greedy, dtype=np.int64)
    d = depths(parent)
    n = parent.shape[0]
    ok = np.zeros(n, dtype=bool)
    ok[0] = True
    for v in range(1, n):
        p = parent[v]
        ok[v] = bool(ok[p]) and draft[v] == greedy[p]
    end = 0
    for v in range(1, n):
        if ok[v] and d[v] > d[end]:
            end = v
    path = []
    v = end
    while v != 0:
        path.append(v)
        v = int(parent[v])
    return end, path[::-1], int(greedy[end])


def admissible_argmax(C, T):
    """Per row, the indices a correct fp32 evaluation of the product may return as its argmax:
    every n whose exact logit C[n] lies within T[n] + T[n*] of the exact maximum C[n*] (T the
    per-element error bound), since two values that close may swap order after rounding."""
    C = np.asarray(C, dtype=np.float64)
    T = np.asarray(T, dtype=np.float64)
    out = []
    for m in range(C.shape[0]):
        star = int(np.argmax(C[m]))
        out.append(set(np.nonzero(C[m] >= C[m, star] - (T[m] + T[m, star]))[0].tolist()))
    return out
