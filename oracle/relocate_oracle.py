"""CPU oracle for Tier-1 KV relocation (live defragmentation of a request's prefix rows).

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only the
tests, the smoke check and the benchmark's CPU-baseline leg may call it.  It shares
no code with the HIP path.

What the pages fix: the "Chunk 66.0" summary has the user direct work on K/V
defragmentation for the scattered page_size=1 pool; the "Chunk 66.1" summary keeps
per-request KV contiguous at allocation time (Tier 0) and defers Tier 1, the live
relocation of rows that are already scattered.  The pages give no further detail,
so the operation below is this library's reading of "live relocation" (each point
is listed among the readings of the design notes):

* The caller picks, per request b, the first slot dst_b of a free run of P_b pool
  slots, or dst_b < 0 to leave b alone.
* For every relocated request and every prefix position j < P_b, columns 0..575 of
  pool row kv_indices[off_b + j] are copied to pool row dst_b + j, and
  kv_indices[off_b + j] becomes dst_b + j.  Tree-node slots are not moved.
* The move is all or nothing.  It is refused (nothing copied, nothing rewritten)
  when any of these holds, each reported by its own error bit:
    - a prefix length outside [0, max_prefix]                    (ERR_BAD_PREFIX)
    - an index of the batch (prefix or tree) outside the pool    (ERR_BAD_INDEX)
    - a destination run that leaves the pool, overlaps another destination run,
      or contains a slot that some index of the batch refers to, other than a row
      that already sits at its own destination                  (ERR_CONFLICT)
  A row whose current slot equals its destination needs no copy and is allowed.
  With these rules no copied row is overwritten before it is read, so the result
  does not depend on the order of the copies.

Pinned in tests/test_relocate_oracle.py against facts that do not come from this
module: the verify attention is unchanged by a relocation (a permutation of the
pool slots), the relocated prefixes are contiguous runs, and each refusal case
leaves the inputs untouched.
"""

from __future__ import annotations

import numpy as np

LATENT = 576

ERR_BAD_INDEX = 0x2
ERR_BAD_PREFIX = 0x4
ERR_CONFLICT = 0x8


def segment_offsets(prefix_lens, tree_nodes: int) -> np.ndarray:
    """off_b: start of request b's segment, the exclusive prefix sum of P_b + T."""
    lens = np.asarray(prefix_lens, dtype=np.int64) + int(tree_nodes)
    return np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)


def relocation_errors(kv_indices, prefix_lens, tree_nodes: int, dst_start, pool_slots: int,
                      max_prefix: int) -> int:
    """The refusal bits of a relocation request (0: it may proceed).

    A bad prefix length is reported alone (the segments can no longer be located).
    Otherwise every cause found sets its bit: out-of-pool indices (ERR_BAD_INDEX,
    and they refer to no slot), and destination runs that leave the pool, overlap
    each other or contain a slot still in use (ERR_CONFLICT)."""
    plens = [int(p) for p in np.asarray(prefix_lens).tolist()]
    if any(p < 0 or p > max_prefix for p in plens):
        return ERR_BAD_PREFIX
    err = 0
    idx = np.asarray(kv_indices, dtype=np.int64)
    offs = segment_offsets(plens, tree_nodes)
    claimed = {}  # destination slot -> (request, prefix position) that moves there
    for b, p in enumerate(plens):
        dst = int(dst_start[b])
        if dst < 0:
            continue
        if dst + p > pool_slots:
            err |= ERR_CONFLICT  # this request is then not moved, its rows stay in use
            continue
        for j in range(p):
            if dst + j in claimed:
                err |= ERR_CONFLICT  # two destination runs overlap
            claimed[dst + j] = (b, j)
    for b, p in enumerate(plens):
        for k in range(p + tree_nodes):
            s = int(idx[offs[b] + k])
            if s < 0 or s >= pool_slots:
                err |= ERR_BAD_INDEX
                continue
            if s in claimed and not (k < p and claimed[s] == (b, k)):
                err |= ERR_CONFLICT  # a destination slot still holds a row in use
    return err


def relocate(pool, kv_indices, prefix_lens, tree_nodes: int, dst_start, max_prefix: int):
    """Returns (new_pool, new_kv_indices, error_bits).  On refusal the copies are unchanged."""
    pool = np.array(pool, copy=True)
    idx = np.array(kv_indices, copy=True)
    err = relocation_errors(idx, prefix_lens, tree_nodes, dst_start, pool.shape[0], max_prefix)
    if err:
        return pool, idx, err
    old_pool = pool.copy()
    offs = segment_offsets(prefix_lens, tree_nodes)
    for b, p in enumerate(np.asarray(prefix_lens).tolist()):
        dst = int(dst_start[b])
        if dst < 0:
            continue
        for j in range(int(p)):
            src = int(idx[offs[b] + j])
            pool[dst + j, :LATENT] = old_pool[src, :LATENT]
            idx[offs[b] + j] = dst + j
    return pool, idx, 0
