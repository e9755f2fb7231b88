"""Pins of the tree-verification oracle (oracle/tree.py) against hand-worked trees, an exhaustive
root-path search, the linear-chain special case and degenerate trees (CPU only)."""
import os

import numpy as np
import pytest

from oracle import tree as TR

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_accept.txt")


def _ints(field):
    return [int(x) for x in field.split()]


def golden_cases():
    out = []
    for line in open(GOLDEN):
        if not line.strip() or line.startswith("#"):
            continue
        name, par, dr, gr, end, path, bonus = [f.strip() for f in line.split("|")]
        out.append((name, _ints(par), _ints(dr), _ints(gr), int(end), _ints(path), int(bonus)))
    return out


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c[0])
def test_hand_worked_trees(case):
    _, parent, draft, greedy, end, path, bonus = case
    assert TR.accept(parent, draft, greedy) == (end, path, bonus)


def brute_force(parent, draft, greedy):
    """Every node's root path is walked explicitly; a node is reachable when every edge on its
    path carries the parent's greedy token; the deepest reachable node (lowest index) wins."""
    n = len(parent)
    best, best_path = 0, []
    for v in range(n):
        path, u, good = [], v, True
        while u != 0:
            if draft[u] != greedy[parent[u]]:
                good = False
            path.append(u)
            u = parent[u]
        if good and len(path) > len(best_path):
            best, best_path = v, path[::-1]
    return best, best_path, greedy[best]


def random_tree(rng, n, vocab):
    parent = [-1] + [int(rng.integers(0, v)) for v in range(1, n)]
    greedy = rng.integers(0, vocab, size=n)
    draft = rng.integers(0, vocab, size=n)
    # make matches common: most drafts copy the parent's greedy token
    for v in range(1, n):
        if rng.random() < 0.6:
            draft[v] = greedy[parent[v]]
    return parent, draft.tolist(), greedy.tolist()


def test_matches_exhaustive_search_on_random_trees():
    rng = np.random.default_rng(12)
    for _ in range(3000):
        n = int(rng.integers(1, 17))
        parent, draft, greedy = random_tree(rng, n, vocab=int(rng.integers(2, 6)))
        assert TR.accept(parent, draft, greedy) == brute_force(parent, draft, greedy)


def test_linear_chain_is_longest_matching_prefix():
    """A chain (parent[v] = v - 1) is linear speculative decoding: the accepted length is the
    number of leading positions where the draft equals the target's previous greedy token."""
    rng = np.random.default_rng(3)
    for _ in range(500):
        n = int(rng.integers(1, 17))
        greedy = rng.integers(0, 3, size=n)
        draft = np.concatenate([[0], np.where(rng.random(n - 1) < 0.7, greedy[:-1], rng.integers(0, 3, size=n - 1))])
        match = draft[1:] == greedy[:-1]
        L = int(np.cumprod(match).sum()) if n > 1 else 0
        end, path, bonus = TR.accept(list(range(-1, n - 1)), draft, greedy)
        assert end == L and path == list(range(1, L + 1)) and bonus == greedy[L]


def test_degenerate_trees_and_errors():
    assert TR.accept([-1], [0], [3]) == (0, [], 3)
    # a star of 15 children, none matching
    assert TR.accept([-1] + [0] * 15, [0] + [1] * 15, [2] * 16) == (0, [], 2)
    # a star where only child 7 matches
    draft = [0] + [1] * 15
    draft[7] = 2
    assert TR.accept([-1] + [0] * 15, draft, [2] * 16) == (7, [7], 2)
    with pytest.raises(ValueError):
        TR.depths([0, 0])
    with pytest.raises(ValueError):
        TR.depths([-1, 1])


def test_greedy_tokens_ties_and_admissible_set():
    C = np.array([[1.0, 3.0, 3.0, 2.0], [0.0, -1.0, 0.0, -2.0]])
    assert TR.greedy_tokens(C).tolist() == [1, 0]
    T = np.full_like(C, 0.01)
    assert TR.admissible_argmax(C, T) == [{1, 2}, {0, 2}]
    T2 = np.full_like(C, 0.6)
    assert TR.admissible_argmax(C, T2)[0] == {1, 2, 3}
