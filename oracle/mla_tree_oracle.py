"""CPU fp64 oracle for DDTree speculative-decode verify attention (absorbed MLA).

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only the
tests, the smoke check and the benchmark's CPU-baseline leg may call it.  It is a
plain, slow, obviously correct restatement of what the verify step computes, and
it shares no code with the HIP path.

What is computed (readings of the pages, in order):

* "Chunk 66.0" (magik.net llmopt, segment 66), summary paragraph: the DDTree
  verify attention is MLA attention over a KV pool with page_size=1, i.e. every
  key is one pool row addressed through a per-request token-index table; the
  owned kernel is checked for token-exact agreement with a naive reference.
  This module is that naive reference, in float64.
* Absorbed (latent) MLA: all H heads of one tensor-parallel rank score against
  the same 576-wide latent row (512 latent + 64 rope columns) and read their
  value from its first 512 columns.
* Tree verification: node i of a request's draft tree sees every prefix token
  of its request, every ancestor of i in the tree, and i itself.
* Index layout: request b owns kv_indices[off_b : off_b + P_b + T]; the first
  P_b entries are its prefix slots in order, the next T are the slots holding
  the latents of tree nodes 0..T-1; off_b is the exclusive prefix sum of
  P_b + T over the requests.
* Rows of q are ordered (request, node, head): q[(b*T + i), h, :].
* lse is the natural log of the sum of exp(score) over the visible keys.

For request b, node i, head h, with sigma the softmax scale:

    Vis(b, i)  = prefix slots of b  ++  tree slots of anc*(i)
    s_j        = sigma * sum_{d < 576} q[b, i, h, d] * KV[j, d]
    lse[b,i,h] = m + ln sum_{j in Vis} exp(s_j - m),   m = max_j s_j
    out[b,i,h] = sum_{j in Vis} exp(s_j - lse) * KV[j, 0:512]

Every bf16 input is widened exactly to float64 before any arithmetic.
All functions here have independent pins in tests/test_oracle.py.
"""

from __future__ import annotations

import math

import numpy as np

LATENT = 576
VDIM = 512


# --------------------------------------------------------------------------- inputs

def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64: the bits are the top half of a float32."""
    bits = np.asarray(bits, dtype=np.uint16)
    as_u32 = bits.astype(np.uint32) << np.uint32(16)
    return as_u32.view(np.float32).astype(np.float64)


def validate_parents(parents) -> None:
    """A tree in topological order: every parent is -1 (a root) or an earlier node."""
    for i, p in enumerate(np.asarray(parents).tolist()):
        if not (-1 <= p < i):
            raise ValueError(f"node {i} has parent {p}; need -1 <= parent < node")


def ancestors_with_self(parents, i: int) -> list[int]:
    """anc*(i): node i, its parent, its parent's parent, ... up to a root, returned in ascending order."""
    parents = np.asarray(parents).tolist()
    chain = []
    node = i
    while node != -1:
        if not (-1 <= parents[node] < node):
            raise ValueError(f"node {node} has parent {parents[node]}")
        chain.append(node)
        node = parents[node]
    return sorted(chain)


def ancestor_masks(parents) -> np.ndarray:
    """Bit j of mask[i] is set iff tree node j is in anc*(i) (T <= 64 nodes, one uint64 per node)."""
    parents = np.asarray(parents)
    t = len(parents)
    if t > 64:
        raise ValueError("one 64-bit mask word holds at most 64 nodes")
    validate_parents(parents)
    masks = np.zeros(t, dtype=np.uint64)
    for i in range(t):
        word = 0
        for a in ancestors_with_self(parents, i):
            word |= 1 << a
        masks[i] = np.uint64(word)
    return masks


def ancestor_mask_words(parents) -> np.ndarray:
    """The same masks for any T, as ceil(T / 64) uint64 words per node: bit j % 64 of word
    j // 64 of row i is set iff node j is in anc*(i)."""
    parents = np.asarray(parents)
    t = len(parents)
    validate_parents(parents)
    words = np.zeros((t, -(-t // 64)), dtype=np.uint64)
    for i in range(t):
        for a in ancestors_with_self(parents, i):
            words[i, a // 64] |= np.uint64(1 << (a % 64))
    return words


def request_offsets(prefix_lens, tree_nodes: int) -> np.ndarray:
    """off_b: start of request b's segment in kv_indices (exclusive prefix sum of P_b + T)."""
    offs = np.zeros(len(prefix_lens), dtype=np.int64)
    running = 0
    for b, p in enumerate(np.asarray(prefix_lens).tolist()):
        offs[b] = running
        running += int(p) + tree_nodes
    return offs


def expand_block_table(kv_indices, prefix_lens, tree_nodes: int, page_size: int) -> np.ndarray:
    """Per-token index list of a batch whose prefixes are paged.

    A paged layout is this library's reading of a block table for the same pool (the
    "Chunk 66.0" and "Chunk 66.1" summaries only speak of page_size=1): request b's
    segment holds ceil(P_b / p) page ids, then its T tree slots, and prefix token j lives
    in pool slot page_id[j // p] * p + j % p.  With p = 1 the list is unchanged.
    """
    idx = np.asarray(kv_indices, dtype=np.int64)
    out, pos = [], 0
    for p_b in np.asarray(prefix_lens).tolist():
        n_pages = -(-int(p_b) // page_size)
        table = idx[pos:pos + n_pages]
        j = np.arange(int(p_b), dtype=np.int64)
        out.append(table[j // page_size] * page_size + j % page_size)
        out.append(idx[pos + n_pages:pos + n_pages + tree_nodes])
        pos += n_pages + tree_nodes
    return np.concatenate(out).astype(np.int64) if out else np.zeros(0, dtype=np.int64)


def visible_slots(kv_indices, prefix_lens, tree_parent, b: int, i: int) -> np.ndarray:
    """Pool rows node i of request b attends to, as a list: the prefix slots, then anc*(i)'s slots."""
    tree_parent = np.asarray(tree_parent)
    t = tree_parent.shape[1]
    off = int(request_offsets(prefix_lens, t)[b])
    p = int(prefix_lens[b])
    seg = np.asarray(kv_indices)[off:off + p + t]
    anc = ancestors_with_self(tree_parent[b], i)
    return np.concatenate([seg[:p], seg[p + np.asarray(anc, dtype=np.int64)]]).astype(np.int64)


# --------------------------------------------------------------------------- attention

def attention_over_slots(q_rows, pool, slots, sm_scale: float):
    """Softmax attention of query rows (float64 [R, 576]) over one explicit list of pool rows.

    Returns (out [R, 512], lse [R]).  An empty list gives lse = -inf and out = 0
    (the empty sum), which is what merging by LSE needs.
    """
    q_rows = np.atleast_2d(np.asarray(q_rows, dtype=np.float64))
    slots = np.asarray(slots, dtype=np.int64)
    r = q_rows.shape[0]
    if slots.size == 0:
        return np.zeros((r, VDIM)), np.full(r, -np.inf)
    kv = bf16_to_f64(np.asarray(pool)[slots, :LATENT])  # [N, 576]
    s = sm_scale * (q_rows @ kv.T)  # [R, N]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(z))[:, 0]
    w = e / z
    return w @ kv[:, :VDIM], lse


def verify_attention(q, pool, kv_indices, prefix_lens, tree_parent, sm_scale: float,
                     *, nodes_per_chunk: int = 16, nodes=None):
    """Tree-verify attention for a batch, in float64.

    q: uint16 bf16 bits [B*T, H, 576]; pool: uint16 [slots, row_stride >= 576];
    kv_indices: int [sum_b(P_b + T)]; prefix_lens: int [B]; tree_parent: int [B, T].
    Returns out float64 [B*T, H, 512] and lse float64 [B*T, H].

    For each request, the scores of every node's rows against the shared prefix
    keys are one matrix product (rows are independent, so this is the per-row
    definition evaluated for several rows at once); the ancestor keys of each node
    are then appended to that node's score list, and softmax, lse and the weighted
    sum of V rows follow the definition row by row.

    ``nodes``: optional iterable of (b, i) pairs; only those rows are computed and
    every other row of the result is NaN (for sampled checks of large batches).
    """
    q = np.asarray(q)
    pool = np.asarray(pool)
    tree_parent = np.asarray(tree_parent)
    prefix_lens = np.asarray(prefix_lens)
    kv_indices = np.asarray(kv_indices)
    bsz, t = tree_parent.shape
    h = q.shape[1]
    assert q.shape == (bsz * t, h, LATENT), q.shape
    if len(kv_indices) != int(prefix_lens.sum()) + bsz * t:
        raise ValueError("kv_indices length must be sum(P_b) + B*T")
    if np.any(prefix_lens < 0):
        raise ValueError("negative prefix length")
    offs = request_offsets(prefix_lens, t)
    fill = 0.0 if nodes is None else np.nan
    out = np.full((bsz * t, h, VDIM), fill)
    lse = np.full((bsz * t, h), fill)
    wanted = None if nodes is None else {(int(b), int(i)) for b, i in nodes}
    for b in range(bsz):
        validate_parents(tree_parent[b])
        if wanted is not None and not any(bb == b for bb, _ in wanted):
            continue
        p = int(prefix_lens[b])
        seg = kv_indices[offs[b]:offs[b] + p + t].astype(np.int64)
        k_pre = bf16_to_f64(pool[seg[:p], :LATENT])  # [P, 576]
        k_tree = bf16_to_f64(pool[seg[p:], :LATENT])  # [T, 576]
        sel = list(range(t)) if wanted is None else sorted(i for bb, i in wanted if bb == b)
        for c0 in range(0, len(sel), nodes_per_chunk):
            chunk = sel[c0:c0 + nodes_per_chunk]
            qb = bf16_to_f64(q[b * t + np.asarray(chunk)])  # [n, H, 576]
            s_pre = sm_scale * (qb.reshape(-1, LATENT) @ k_pre.T)  # [n*H, P]
            s_pre = s_pre.reshape(len(chunk), h, p)
            for ci, i in enumerate(chunk):
                anc = np.asarray(ancestors_with_self(tree_parent[b, :], i), dtype=np.int64)
                k_anc = k_tree[anc]  # [a, 576]
                s = np.concatenate([s_pre[ci], sm_scale * (qb[ci] @ k_anc.T)], axis=1)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                z = e.sum(axis=1, keepdims=True)
                w = e / z
                row = b * t + i
                lse[row] = (m + np.log(z))[:, 0]
                out[row] = w[:, :p] @ k_pre[:, :VDIM] + w[:, p:] @ k_anc[:, :VDIM]
    return out, lse


def node_offsets(tree_lens) -> np.ndarray:
    """First packed row (node) of each request when requests have T_b = tree_lens[b] nodes:
    the exclusive prefix sum of tree_lens."""
    tl = np.asarray(tree_lens, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(tl)[:-1]]).astype(np.int64)


def verify_attention_ragged(q, pool, kv_indices, prefix_lens, tree_lens, tree_parent, sm_scale: float):
    """Tree-verify attention for a batch whose requests draft trees of different sizes.

    Request b has T_b = tree_lens[b] >= 1 nodes.  Rows are packed request after request:
    node i of request b is row n_b + i (n_b = node_offsets(tree_lens)[b]) of q [sum T_b, H, 576]
    and of the results; tree_parent [sum T_b] holds, at n_b + i, the parent of node i within
    its request (-1 for a root, else an earlier node of the same request).  Request b owns
    kv_indices[off_b : off_b + P_b + T_b], its prefix slots then the slots of its tree nodes,
    with off_b the exclusive prefix sum of P_b + T_b.  Each request is the definition above
    with T = T_b (no node of one request sees another request's nodes), so the result is the
    per-request attention written into the packed rows.
    Returns out float64 [sum T_b, H, 512] and lse float64 [sum T_b, H].
    """
    q = np.asarray(q)
    tree_lens = np.asarray(tree_lens, dtype=np.int64)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    kv_indices = np.asarray(kv_indices)
    tree_parent = np.asarray(tree_parent)
    if np.any(tree_lens < 1):
        raise ValueError("every request needs at least one tree node")
    total = int(tree_lens.sum())
    if q.shape[0] != total or len(tree_parent) != total:
        raise ValueError("q and tree_parent must hold sum(tree_lens) rows")
    if len(kv_indices) != int(prefix_lens.sum() + tree_lens.sum()):
        raise ValueError("kv_indices length must be sum(P_b + T_b)")
    h = q.shape[1]
    out = np.zeros((total, h, VDIM))
    lse = np.zeros((total, h))
    nodes = node_offsets(tree_lens)
    off = 0
    for b in range(len(tree_lens)):
        p, t, n = int(prefix_lens[b]), int(tree_lens[b]), int(nodes[b])
        o, l = verify_attention(q[n:n + t], pool, kv_indices[off:off + p + t], np.array([p]),
                                tree_parent[None, n:n + t], sm_scale)
        out[n:n + t], lse[n:n + t] = o, l
        off += p + t
    return out, lse


def attention_weights(q, pool, kv_indices, prefix_lens, tree_parent, sm_scale: float, b: int, i: int):
    """Softmax weights of node i of request b over Vis(b, i), float64 [H, |Vis|] (for the row-sum pin)."""
    t = np.asarray(tree_parent).shape[1]
    slots = visible_slots(kv_indices, prefix_lens, tree_parent, b, i)
    kv = bf16_to_f64(np.asarray(pool)[slots, :LATENT])
    qi = bf16_to_f64(np.asarray(q)[b * t + i])
    s = sm_scale * (qi @ kv.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def lse_merge(outs, lses):
    """Combine attention results over disjoint parts of one key list.

    With lse = logsumexp over parts of lse_u, the merged output is
    sum_u exp(lse_u - lse) * out_u.  Parts with lse_u = -inf (empty) contribute
    nothing.  outs: list of [R, 512]; lses: list of [R].
    """
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lses])  # [U, R]
    O = np.stack([np.asarray(x, dtype=np.float64) for x in outs])  # [U, R, 512]
    m = L.max(axis=0)
    finite = np.isfinite(m)
    safe_m = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(L), np.exp(L - safe_m), 0.0)
    z = w.sum(axis=0)
    lse = np.where(finite, safe_m + np.log(np.where(finite, z, 1.0)), -np.inf)
    coef = np.where(finite, w / np.where(finite, z, 1.0), 0.0)
    out = np.einsum("ur,urd->rd", coef, O)
    return out, lse


# --------------------------------------------------------------------------- brute force

def brute_force_verify_attention(q, pool, kv_indices, prefix_lens, tree_parent, sm_scale: float):
    """Same result with nothing but Python loops and math.fsum; for tiny inputs only."""
    q = np.asarray(q)
    pool = np.asarray(pool)
    tree_parent = np.asarray(tree_parent).tolist()
    prefix_lens = [int(x) for x in np.asarray(prefix_lens).tolist()]
    kv_indices = [int(x) for x in np.asarray(kv_indices).tolist()]
    bsz = len(tree_parent)
    t = len(tree_parent[0])
    h = q.shape[1]

    def widen(u16):
        return float(np.frombuffer(np.uint32(int(u16) << 16).tobytes(), dtype=np.float32)[0])

    out = np.zeros((bsz * t, h, VDIM))
    lse = np.zeros((bsz * t, h))
    off = 0
    for b in range(bsz):
        p = prefix_lens[b]
        seg = kv_indices[off:off + p + t]
        off += p + t
        for i in range(t):
            keys = list(seg[:p])
            node = i
            chain = []
            while node != -1:
                chain.append(node)
                node = tree_parent[b][node]
            for a in sorted(chain):
                keys.append(seg[p + a])
            rows = [[widen(x) for x in pool[k, :LATENT]] for k in keys]
            for hh in range(h):
                qv = [widen(x) for x in q[b * t + i, hh]]
                s = [sm_scale * math.fsum(qv[d] * row[d] for d in range(LATENT)) for row in rows]
                m = max(s)
                z = math.fsum(math.exp(x - m) for x in s)
                l = m + math.log(z)
                lse[b * t + i, hh] = l
                w = [math.exp(x - l) for x in s]
                for d in range(VDIM):
                    out[b * t + i, hh, d] = math.fsum(w[j] * rows[j][d] for j in range(len(rows)))
    return out, lse
