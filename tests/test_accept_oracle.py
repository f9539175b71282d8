"""Pins of the greedy-acceptance oracle (oracle/accept_oracle.py) on the CPU.

Expected values come from elsewhere: brute force over every path of the tree with numpy's
own argmax (with distinct sibling tokens the greedy walk must find the unique longest
matching path), a hand-derived tree, and the stated argmax rules checked by hand.
"""

import itertools

import numpy as np
import pytest

from oracle import accept_oracle as acc
from workloads import synth


def all_paths(parents):
    """Every downward path that starts at a first-level node (including the empty one)."""
    t = len(parents)
    out = [[]]
    frontier = [[i] for i in range(t) if parents[i] == -1]
    while frontier:
        out += frontier
        frontier = [p + [c] for p in frontier for c in range(t) if parents[c] == p[-1]]
    return out


def brute_force(logits, tokens, parents):
    best = []
    for path in all_paths(parents):
        rows = [0] + [1 + n for n in path[:-1]]
        if all(tokens[n] == int(np.argmax(logits[r])) for n, r in zip(path, rows)) and len(path) > len(best):
            best = path
    bonus = int(np.argmax(logits[1 + best[-1]] if best else logits[0]))
    return best, bonus


@pytest.mark.parametrize("seed,t,vocab", [(0, 8, 16), (1, 16, 5), (2, 33, 50), (3, 64, 200), (4, 1, 3)])
def test_greedy_path_is_the_longest_matching_path(seed, t, vocab):
    cfg = synth.accept_config(seed, batch=6, tree_nodes=t, vocab=vocab)
    lens, accd, bonus, err = acc.accept(cfg["logits"], cfg["draft_tokens"], cfg["tree_parent"])
    assert err == 0
    for b in range(6):
        path, g = brute_force(cfg["logits"][b], cfg["draft_tokens"][b], cfg["tree_parent"][b].tolist())
        assert accd[b, :lens[b]].tolist() == path and bonus[b] == g
        assert len(path) >= len(cfg["planted"][b])  # the planted path matches (it may continue)
        assert all(x == -1 for x in accd[b, lens[b]:])


def test_hand_derived_tree():
    parents = [-1, 0, 1, 2, 0, 4, 1, 6]
    tokens = [5, 6, 7, 8, 9, 10, 11, 12]
    logits = np.zeros((9, 16), dtype=np.float32)
    logits[0, 5] = 1      # first level: node 0 (token 5)
    logits[1, 9] = 1      # after node 0: children 1 (6) and 4 (9) -> node 4
    logits[5, 10] = 1     # after node 4: child 5 (10)
    logits[6, 3] = 1      # after node 5: no child, bonus token 3
    path, g, err = acc.accept_one(logits, tokens, parents)
    assert (path, g, err) == ([0, 4, 5], 3, 0)
    logits[0, 5] = 0
    logits[0, 2] = 1      # no first-level node has token 2: nothing accepted
    assert acc.accept_one(logits, tokens, parents) == ([], 2, 0)


def test_duplicate_sibling_tokens_take_the_lowest_index():
    parents = [-1, 0, 0, 1, 2]
    tokens = [1, 4, 4, 7, 8]
    logits = np.zeros((6, 10), dtype=np.float32)
    logits[0, 1] = 1
    logits[1, 4] = 1
    logits[3, 8] = 1      # after node 2 the walk could go on to node 4, but node 1 is taken
    path, g, _ = acc.accept_one(logits, tokens, parents)
    assert path == [0, 1] and g == 0


def test_argmax_rules():
    nan, inf = float("nan"), float("inf")
    assert acc.argmax_row([1.0, 3.0, 3.0, 2.0]) == 1          # lowest index on ties
    assert acc.argmax_row([nan, 0.5, nan, 0.7]) == 3          # NaN ignored
    assert acc.argmax_row([nan, nan]) == 0                    # NaN only
    assert acc.argmax_row([nan, -inf, -inf]) == 1             # -inf ranks above NaN
    assert acc.argmax_row([-0.0, 0.0]) == 0                   # equal values


def test_invalid_tree_accepts_nothing():
    logits = np.zeros((4, 5), dtype=np.float32)
    logits[0, 2] = 1
    path, g, err = acc.accept_one(logits, [2, 3, 4], [-1, 2, 0])
    assert path == [] and g == 2 and err == acc.ERR_BAD_PARENT
