"""CPU oracle for greedy acceptance of a verified draft tree.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only the
tests, the smoke check and the benchmark's CPU-baseline leg may call it.  It shares
no code with the HIP path.

What the pages fix: the verify pass scores every node of the draft tree in one target
step, and the step commits the drafted tokens the target agrees with plus one token of
its own; the "Chunk 66.0" summary reports commit lengths of 7-8 on predictable text and
of 1 on hard text.  The rule below is this library's reading of that step (it is listed
among the readings of the design notes):

* logits[b, 0] are the target's logits at the position before the tree; logits[b, 1 + i]
  are its logits after tree node i.  Nodes with parent -1 are the tree's first level.
* Walk from the position before the tree: g = argmax of the current row; the next node is
  the lowest-index child (a first-level node at the start) whose draft token is g.  Accept
  it and continue from its row; stop when no child matches.
* The bonus token is the argmax of the last row visited.  The step commits the accepted
  nodes' tokens and then the bonus token (accepted + 1 tokens).
* argmax: the largest value, the lowest index among equal values; NaN ranks below every
  number (a row of NaN only gives index 0).
* An invalid tree (a parent outside [-1, node)) accepts nothing and reports ERR_BAD_PARENT;
  its bonus token is still the argmax of row 0.

Pinned in tests/test_accept_oracle.py: brute force over every path of the tree (with
distinct sibling tokens the greedy path is the unique longest matching path), a
hand-derived tree, and the argmax rules.
"""

from __future__ import annotations

import numpy as np

ERR_BAD_PARENT = 0x1


def argmax_row(row) -> int:
    """Index of the largest value, lowest index on ties, NaN below every number."""
    row = np.asarray(row, dtype=np.float64)
    ok = ~np.isnan(row)
    if not ok.any():
        return 0
    best = row[ok].max()
    return int(np.nonzero(ok & (row == best))[0][0])


def valid_tree(parents) -> bool:
    return all(-1 <= int(p) < i for i, p in enumerate(np.asarray(parents).tolist()))


def accept_one(logits, draft_tokens, parents):
    """(accepted node ids in path order, bonus token, error bits) of one request."""
    parents = np.asarray(parents).tolist()
    tokens = np.asarray(draft_tokens).tolist()
    if not valid_tree(parents):
        return [], argmax_row(logits[0]), ERR_BAD_PARENT
    path, node, row = [], -1, 0
    while True:
        g = argmax_row(logits[row])
        nxt = next((i for i, p in enumerate(parents) if p == node and tokens[i] == g), None)
        if nxt is None:
            return path, g, 0
        path.append(nxt)
        node, row = nxt, 1 + nxt


def accept(logits, draft_tokens, tree_parent):
    """Batch form: accept_len [B], accepted [B, T] (-1 padded), bonus [B], error bits (OR)."""
    logits = np.asarray(logits)
    b, t = np.asarray(tree_parent).shape
    lens = np.zeros(b, dtype=np.int32)
    acc = np.full((b, t), -1, dtype=np.int32)
    bonus = np.zeros(b, dtype=np.int32)
    err = 0
    for r in range(b):
        path, g, e = accept_one(logits[r], draft_tokens[r], tree_parent[r])
        lens[r] = len(path)
        acc[r, :len(path)] = path
        bonus[r] = g
        err |= e
    return lens, acc, bonus, err
