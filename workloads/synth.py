"""Seeded workload recipes for DDTree speculative-decode verify attention.

The workloads mirror the long-context decode setting described on the page
"Chunk 66.0" (magik.net llmopt, segment 66, summary paragraph): a draft tree is
verified against a request prefix held in a page_size=1 token pool, for prefixes
from a few thousand up to 185k tokens, with one tensor-parallel rank's share of
heads (8 per rank under TP8, page "Chunk 66.1", summary paragraph).  The pages
carry no prompts, traces or weights, so every value here is synthetic:

* latent KV rows are 576 bf16 wide (512 latent + 64 rope, absorbed MLA), V is
  the first 512 columns;
* q and KV values are N(0, 1) * 0.1 drawn in float32 and rounded to bf16 with
  round-to-nearest-even;
* random draft trees give node i >= 1 a parent drawn uniformly from the earlier
  nodes whose depth is at most 7 (so no node is deeper than 8 edges);
* token indices are drawn without replacement from the pool ("scattered"), or
  laid out as one contiguous run per request ("contiguous", what a defragmented
  allocator produces).

Draw order for every config: tree(s) -> prefix lengths -> indices -> q -> pool.
Arrays use numpy; bf16 values are carried as their uint16 bit patterns.
"""

from __future__ import annotations

import math

import numpy as np

LATENT_DIM = 576  # 512 latent + 64 rope columns per KV row
V_DIM = 512  # V is the first 512 columns of a KV row
DEFAULT_SCALE = 1.0 / math.sqrt(192.0)

# name, batch, prefix (int or ("loguniform", lo, hi)), tree nodes, heads, pool slots,
# tree kind, index layout.  Keys 0-4 are the verify workloads; 5 and 6 are the two
# HBM-bound shapes (small trees) used to show scattered-read bandwidth.
CONFIGS = {
    0: dict(name="tiny_p256_t8_h8", batch=1, prefix=256, tree_nodes=8, heads=8, slots=512,
            tree="tiny", indices="contiguous"),
    1: dict(name="p4096_t64_h8", batch=1, prefix=4096, tree_nodes=64, heads=8, slots=262144,
            tree="random", indices="scattered"),
    2: dict(name="p65536_t64_h8", batch=1, prefix=65536, tree_nodes=64, heads=8, slots=262144,
            tree="random", indices="scattered"),
    3: dict(name="p185000_t64_h8", batch=1, prefix=185000, tree_nodes=64, heads=8, slots=262144,
            tree="random", indices="scattered"),
    4: dict(name="b8_ploguniform_t32_h16", batch=8, prefix=("loguniform", 1024, 131072),
            tree_nodes=32, heads=16, slots=1048576, tree="random", indices="scattered"),
    5: dict(name="p185000_t8_h8", batch=1, prefix=185000, tree_nodes=8, heads=8, slots=262144,
            tree="random", indices="scattered"),
    6: dict(name="p185000_t16_h8", batch=1, prefix=185000, tree_nodes=16, heads=8, slots=262144,
            tree="random", indices="scattered"),
}

BF16_QNAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); NaN stays a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # in 32 bits: for every non-NaN pattern u + 0x8000 stays below 2^32 (the largest finite
    # values round to infinity, as they should); NaN patterns are replaced below
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        sign = ((u >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint16)
        rounded = np.where(nan, sign | BF16_QNAN, rounded)
    return rounded


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def tiny_tree() -> np.ndarray:
    """The 8-node tree of the tiny workload: parents [-1, 0, 1, 2, 0, 4, 1, 6]."""
    return np.array([-1, 0, 1, 2, 0, 4, 1, 6], dtype=np.int32)


def chain_tree(t: int) -> np.ndarray:
    """A single path: node i's parent is i - 1."""
    return np.arange(-1, t - 1, dtype=np.int32)


def tree_depths(parents) -> np.ndarray:
    """Edge depth of each node (roots have depth 0); parents must precede children."""
    parents = np.asarray(parents)
    depth = np.zeros(len(parents), dtype=np.int64)
    for i, p in enumerate(parents):
        depth[i] = 0 if p < 0 else depth[p] + 1
    return depth


def random_tree(rng: np.random.Generator, t: int, max_depth: int = 8) -> np.ndarray:
    """Node 0 is the root; node i >= 1 takes a parent uniformly among earlier nodes of depth < max_depth."""
    parents = np.full(t, -1, dtype=np.int32)
    depth = np.zeros(t, dtype=np.int64)
    for i in range(1, t):
        cand = np.nonzero(depth[:i] < max_depth)[0]
        p = int(cand[rng.integers(0, len(cand))])
        parents[i] = p
        depth[i] = depth[p] + 1
    return parents


def _draw_prefix_lens(rng, spec, batch):
    if isinstance(spec, tuple):
        kind, lo, hi = spec
        assert kind == "loguniform"
        u = rng.uniform(math.log(lo), math.log(hi), size=batch)
        return np.clip(np.floor(np.exp(u)), lo, hi).astype(np.int32)
    return np.full(batch, int(spec), dtype=np.int32)


def _bf16_normal(rng, shape, scale=0.1, chunk_rows=65536):
    """N(0,1)*scale as bf16 bits, drawn row-chunk by row-chunk along axis 0."""
    out = np.empty(shape, dtype=np.uint16)
    n = shape[0]
    for s in range(0, n, chunk_rows):
        e = min(n, s + chunk_rows)
        x = rng.standard_normal((e - s,) + tuple(shape[1:]), dtype=np.float32)
        x *= np.float32(scale)
        out[s:e] = f32_to_bf16_bits(x)
    return out


def make_config(i: int, seed: int | None = None, *, variant: str | None = None,
                prefix_override=None, slots_override: int | None = None,
                row_stride: int = LATENT_DIM) -> dict:
    """Build workload ``i`` from ``CONFIGS`` with ``numpy.random.default_rng(seed or i)``.

    Returns a dict with ``q`` (uint16 [B*T, H, 576]), ``pool`` (uint16 [slots, row_stride]),
    ``kv_indices`` (int32, per request: P_b prefix slots then T tree slots, requests back to
    back), ``prefix_lens`` (int32 [B]), ``tree_parent`` (int32 [B, T]) and the sizes.
    ``variant`` applies one of the transformations in ``VARIANTS`` afterwards.
    """
    spec = dict(CONFIGS[i])
    rng = np.random.default_rng(i if seed is None else seed)
    b, t, h = spec["batch"], spec["tree_nodes"], spec["heads"]
    slots = slots_override if slots_override is not None else spec["slots"]

    # trees
    if spec["tree"] == "tiny":
        parents = np.stack([tiny_tree() for _ in range(b)])
    else:
        parents = np.stack([random_tree(rng, t) for _ in range(b)])
    # prefix lengths
    pspec = prefix_override if prefix_override is not None else spec["prefix"]
    prefix_lens = _draw_prefix_lens(rng, pspec, b)
    total = int(prefix_lens.sum()) + b * t
    if total > slots:
        raise ValueError(f"workload needs {total} token slots, pool has {slots}")
    # indices
    if spec["indices"] == "contiguous":
        kv_indices = np.arange(total, dtype=np.int32)
    else:
        kv_indices = rng.choice(slots, size=total, replace=False).astype(np.int32)
    # values
    q = _bf16_normal(rng, (b * t, h, LATENT_DIM))
    pool = _bf16_normal(rng, (slots, LATENT_DIM))
    if row_stride != LATENT_DIM:
        if row_stride < LATENT_DIM:
            raise ValueError("row_stride must be >= 576")
        padded = np.full((slots, row_stride), BF16_QNAN, dtype=np.uint16)
        padded[:, :LATENT_DIM] = pool
        pool = padded
    cfg = dict(name=spec["name"], config=i, seed=(i if seed is None else seed), batch=b,
               tree_nodes=t, heads=h, slots=slots, row_stride=row_stride,
               sm_scale=DEFAULT_SCALE, q=q, pool=pool, kv_indices=kv_indices,
               prefix_lens=prefix_lens, tree_parent=parents.astype(np.int32), variant=None)
    if variant is not None:
        cfg = apply_variant(cfg, variant, rng)
    return cfg


def request_offsets(prefix_lens, tree_nodes) -> np.ndarray:
    """Start of each request's segment in kv_indices (exclusive scan of P_b + T)."""
    seg = np.asarray(prefix_lens, dtype=np.int64) + tree_nodes
    return np.concatenate([[0], np.cumsum(seg)[:-1]]).astype(np.int64)


def _sorted_segments(cfg):
    idx = cfg["kv_indices"].copy()
    offs = request_offsets(cfg["prefix_lens"], cfg["tree_nodes"])
    for b, o in enumerate(offs):
        p = int(cfg["prefix_lens"][b])
        idx[o:o + p] = np.sort(idx[o:o + p])
        idx[o + p:o + p + cfg["tree_nodes"]] = np.sort(idx[o + p:o + p + cfg["tree_nodes"]])
    cfg["kv_indices"] = idx
    return cfg


def _contiguous(cfg):
    total = len(cfg["kv_indices"])
    base = (cfg["slots"] - total) // 2
    cfg["kv_indices"] = (base + np.arange(total)).astype(np.int32)
    return cfg


def _poison_unused(cfg):
    used = np.zeros(cfg["slots"], dtype=bool)
    used[cfg["kv_indices"]] = True
    pool = cfg["pool"].copy()
    pool[~used] = BF16_QNAN
    cfg["pool"] = pool
    return cfg


def _scale_q(cfg, factor):
    q = bf16_bits_to_f32(cfg["q"]) * np.float32(factor)
    cfg["q"] = f32_to_bf16_bits(q)
    return cfg


def _needle(cfg, rng, where):
    """Plant one key that dominates every score it is visible to.

    A random +-1 direction u is drawn; the chosen key row becomes 2u and every q row
    gets 0.5u added, so that key's score is about sm_scale * 576 (about 41.6) above
    the others.  ``where`` is "prefix" (slot at a random prefix position of each
    request) or "tree" (the slot of tree node 1 of each request, visible only to the
    rows of node 1 and its descendants).
    """
    u = np.where(rng.integers(0, 2, size=LATENT_DIM) == 1, 1.0, -1.0).astype(np.float32)
    pool = cfg["pool"].copy()
    offs = request_offsets(cfg["prefix_lens"], cfg["tree_nodes"])
    needles = []
    for b, o in enumerate(offs):
        p = int(cfg["prefix_lens"][b])
        if where == "prefix":
            if p == 0:
                raise ValueError("prefix needle needs a prefix")
            pos = int(o + rng.integers(0, p))
        else:
            pos = int(o + p + min(1, cfg["tree_nodes"] - 1))
        slot = int(cfg["kv_indices"][pos])
        pool[slot, :LATENT_DIM] = f32_to_bf16_bits(2.0 * u)
        needles.append(slot)
    q = bf16_bits_to_f32(cfg["q"]) + 0.5 * u[None, None, :]
    cfg["q"] = f32_to_bf16_bits(q)
    cfg["pool"] = pool
    cfg["needle_slots"] = np.array(needles, dtype=np.int64)
    return cfg


def _prefix_zero(cfg):
    offs = request_offsets(cfg["prefix_lens"], cfg["tree_nodes"])
    t = cfg["tree_nodes"]
    keep = np.concatenate([cfg["kv_indices"][o + p:o + p + t]
                           for o, p in zip(offs, cfg["prefix_lens"])])
    cfg["kv_indices"] = keep.astype(np.int32)
    cfg["prefix_lens"] = np.zeros_like(cfg["prefix_lens"])
    return cfg


def _chain(cfg):
    cfg["tree_parent"] = np.stack([chain_tree(cfg["tree_nodes"])
                                   for _ in range(cfg["batch"])]).astype(np.int32)
    return cfg


def _qzero(cfg):
    cfg["q"] = np.zeros_like(cfg["q"])
    return cfg


def column_scales() -> np.ndarray:
    """Fixed power-of-two scales, 2^-12 .. 2^12, one per V column (see ``_colscale``)."""
    return np.exp2(((np.arange(V_DIM) * 7) % 25) - 12).astype(np.float64)


def _colscale(cfg):
    """Multiply V column d of every pool row by column_scales()[d] and divide q column d
    by it.  Both are exact in bf16 (powers of two), so every score is unchanged and each
    output column is the unscaled one times its scale; the outputs of one row then span
    eight decades."""
    sc = column_scales().astype(np.float32)
    pool = cfg["pool"].copy()
    pool[:, :V_DIM] = f32_to_bf16_bits(bf16_bits_to_f32(pool[:, :V_DIM]) * sc)
    q = bf16_bits_to_f32(cfg["q"])
    q[..., :V_DIM] /= sc
    cfg["q"] = f32_to_bf16_bits(q)
    cfg["pool"] = pool
    return cfg


VARIANTS = ("sorted", "contiguous", "poison_unused", "sharp", "qzero", "needle_prefix",
            "needle_tree", "prefix0", "chain", "colscale")


def plant_unit_end_needles(cfg: dict, split: int, seed: int = 0) -> dict:
    """Plant a dominant key (as in the needle variants) at the last prefix key of every split
    unit of ``split`` tokens: prefix positions min(P_b, (u + 1) * split) - 1 of each request.
    Every row then meets a key far above its running maximum in the last prefix tile of each
    unit, the worst place for a raised softmax reference."""
    rng = np.random.default_rng(2000 + seed)
    u = np.where(rng.integers(0, 2, size=LATENT_DIM) == 1, 1.0, -1.0).astype(np.float32)
    cfg = dict(cfg)
    pool = cfg["pool"].copy()
    offs = request_offsets(cfg["prefix_lens"], cfg["tree_nodes"])
    needles = []
    for b, o in enumerate(offs):
        p = int(cfg["prefix_lens"][b])
        for end in range(split, p + split, split):
            slot = int(cfg["kv_indices"][int(o) + min(p, end) - 1])
            pool[slot, :LATENT_DIM] = f32_to_bf16_bits(2.0 * u)
            needles.append(slot)
    cfg["q"] = f32_to_bf16_bits(bf16_bits_to_f32(cfg["q"]) + 0.5 * u[None, None, :])
    cfg["pool"] = pool
    cfg["needle_slots"] = np.array(needles, dtype=np.int64)
    return cfg


def apply_variant(cfg: dict, variant: str, rng: np.random.Generator | None = None) -> dict:
    """Apply one named transformation (see ``VARIANTS``) to a config built by ``make_config``."""
    cfg = dict(cfg)
    if rng is None:
        rng = np.random.default_rng(1000 + int(cfg["seed"]))
    if variant == "sorted":
        cfg = _sorted_segments(cfg)
    elif variant == "contiguous":
        cfg = _contiguous(cfg)
    elif variant == "poison_unused":
        cfg = _poison_unused(cfg)
    elif variant == "sharp":
        cfg = _scale_q(cfg, 30.0)  # q ~ N(0,1) * 3
    elif variant == "qzero":
        cfg = _qzero(cfg)
    elif variant == "needle_prefix":
        cfg = _needle(cfg, rng, "prefix")
    elif variant == "needle_tree":
        cfg = _needle(cfg, rng, "tree")
    elif variant == "prefix0":
        cfg = _prefix_zero(cfg)
    elif variant == "chain":
        cfg = _chain(cfg)
    elif variant == "colscale":
        cfg = _colscale(cfg)
    else:
        raise ValueError(f"unknown variant {variant!r}")
    cfg["variant"] = variant if cfg.get("variant") is None else cfg["variant"] + "+" + variant
    return cfg


def permute_pool(cfg: dict, rng: np.random.Generator) -> dict:
    """Move every pool row to a new slot and remap the indices to follow it."""
    cfg = dict(cfg)
    perm = rng.permutation(cfg["slots"])  # new slot of old row r is perm[r]
    pool = np.empty_like(cfg["pool"])
    pool[perm] = cfg["pool"]
    cfg["pool"] = pool
    cfg["kv_indices"] = perm[cfg["kv_indices"]].astype(np.int32)
    return cfg


def permute_prefix(cfg: dict, rng: np.random.Generator) -> dict:
    """Shuffle the order of each request's prefix slots (membership unchanged)."""
    cfg = dict(cfg)
    idx = cfg["kv_indices"].copy()
    offs = request_offsets(cfg["prefix_lens"], cfg["tree_nodes"])
    for o, p in zip(offs, cfg["prefix_lens"]):
        seg = idx[o:o + int(p)].copy()
        rng.shuffle(seg)
        idx[o:o + int(p)] = seg
    cfg["kv_indices"] = idx
    return cfg


def small_config(seed: int, *, batch: int, prefix, tree_nodes: int, heads: int, slots: int,
                 tree: str = "random", indices: str = "scattered", max_depth: int = 8,
                 q_scale: float = 0.1, row_stride: int = LATENT_DIM) -> dict:
    """A free-form workload (same recipe as ``make_config``) for tests at chosen sizes.

    ``prefix`` is an int, a list of per-request ints, or ("loguniform", lo, hi).
    """
    rng = np.random.default_rng(seed)
    b, t, h = batch, tree_nodes, heads
    if tree == "chain":
        parents = np.stack([chain_tree(t) for _ in range(b)])
    elif tree == "tiny":
        parents = np.stack([tiny_tree() for _ in range(b)])
    elif tree == "forest":
        # several roots: node i's parent is uniform over {-1} + earlier nodes
        parents = np.stack([np.array([int(rng.integers(-1, i)) for i in range(t)], dtype=np.int32)
                            for _ in range(b)])
    else:
        parents = np.stack([random_tree(rng, t, max_depth) for _ in range(b)])
    if isinstance(prefix, (list, np.ndarray)):
        prefix_lens = np.asarray(prefix, dtype=np.int32)
        assert len(prefix_lens) == b
    else:
        prefix_lens = _draw_prefix_lens(rng, prefix, b)
    total = int(prefix_lens.sum()) + b * t
    if total > slots:
        raise ValueError("pool too small")
    if indices == "contiguous":
        kv_indices = np.arange(total, dtype=np.int32)
    else:
        kv_indices = rng.choice(slots, size=total, replace=False).astype(np.int32)
    q = _bf16_normal(rng, (b * t, h, LATENT_DIM), scale=q_scale)
    pool = _bf16_normal(rng, (slots, LATENT_DIM))
    if row_stride != LATENT_DIM:
        padded = np.full((slots, row_stride), BF16_QNAN, dtype=np.uint16)
        padded[:, :LATENT_DIM] = pool
        pool = padded
    return dict(name=f"small_s{seed}", config=None, seed=seed, batch=b, tree_nodes=t, heads=h,
                slots=slots, row_stride=row_stride, sm_scale=DEFAULT_SCALE, q=q, pool=pool,
                kv_indices=kv_indices, prefix_lens=prefix_lens, tree_parent=parents.astype(np.int32),
                variant=None)


def defrag_config(seed: int, *, batch: int, prefix, tree_nodes: int, heads: int, slots: int,
                  row_stride: int = LATENT_DIM) -> dict:
    """A relocation workload: every index of the batch is drawn (without replacement)
    from the lower half of the pool, and ``dst_start[b]`` is the first slot of a free
    run of P_b slots in the upper half (runs in request order, random gaps between
    them; -1 where P_b = 0)."""
    cfg = small_config(seed, batch=batch, prefix=prefix, tree_nodes=tree_nodes, heads=heads, slots=slots,
                       row_stride=row_stride)
    rng = np.random.default_rng(10_000 + seed)
    half = slots // 2
    total = len(cfg["kv_indices"])
    plens = [int(p) for p in cfg["prefix_lens"]]
    if total > half or sum(plens) > slots - half:
        raise ValueError("pool too small for a relocation workload")
    cfg["kv_indices"] = rng.choice(half, size=total, replace=False).astype(np.int32)
    spare = slots - half - sum(plens)
    gaps = np.sort(rng.integers(0, spare + 1, size=batch))
    gaps = np.diff(np.concatenate([[0], gaps]))
    dst, pos = [], half
    for b, p in enumerate(plens):
        pos += int(gaps[b])
        dst.append(pos if p > 0 else -1)
        pos += p
    cfg["dst_start"] = np.asarray(dst, dtype=np.int32)
    cfg["name"] = f"defrag_s{seed}"
    return cfg


def paged_config(seed: int, *, batch: int, prefix, tree_nodes: int, heads: int, slots: int, page: int,
                 contiguous_pages: bool = False) -> dict:
    """A workload whose prefixes are paged: ``kv_indices`` holds, per request, the page ids of
    its ceil(P_b / page) prefix pages (distinct, drawn from the pages below the top quarter of
    the pool; consecutive from a random start when ``contiguous_pages``), then its T tree
    slots, drawn from the top quarter.  ``page_size`` is recorded in the config."""
    cfg = small_config(seed, batch=batch, prefix=prefix, tree_nodes=tree_nodes, heads=heads, slots=slots)
    rng = np.random.default_rng(20_000 + seed)
    top = slots - slots // 4
    n_pages = [-(-int(p) // page) for p in cfg["prefix_lens"]]
    avail = top // page
    if sum(n_pages) > avail or batch * tree_nodes > slots - top:
        raise ValueError("pool too small for a paged workload")
    if contiguous_pages:
        start = int(rng.integers(0, avail - sum(n_pages) + 1))
        pages = np.arange(start, start + sum(n_pages))
    else:
        pages = rng.choice(avail, size=sum(n_pages), replace=False)
    tree_slots = top + rng.choice(slots - top, size=batch * tree_nodes, replace=False)
    segs, pp = [], 0
    for b, n in enumerate(n_pages):
        segs.append(pages[pp:pp + n])
        segs.append(tree_slots[b * tree_nodes:(b + 1) * tree_nodes])
        pp += n
    cfg["kv_indices"] = np.concatenate(segs).astype(np.int32)
    cfg["page_size"] = page
    cfg["name"] = f"paged{page}_s{seed}"
    return cfg


def accept_config(seed: int, *, batch: int, tree_nodes: int, vocab: int, plant: bool = True) -> dict:
    """Inputs of the acceptance step: a random tree per request (as ``random_tree``), draft
    tokens that differ between siblings, and fp32 logits N(0, 1) of shape [B, T + 1, V].
    With ``plant``, a random path from the first level down is made to match: the logits
    of the row before each of its nodes get +20 at that node's token.  (Where the path
    stops, the next argmax is random and may extend it by chance.)"""
    rng = np.random.default_rng(30_000 + seed)
    t = tree_nodes
    parents = np.stack([random_tree(rng, t) for _ in range(batch)]).astype(np.int32)
    if t > 1:  # some requests get several first-level nodes
        for b in range(0, batch, 2):
            parents[b, int(rng.integers(1, t))] = -1
    tokens = np.zeros((batch, t), dtype=np.int32)
    for b in range(batch):
        for node in range(t):
            sib = [int(tokens[b, j]) for j in range(node) if parents[b, j] == parents[b, node]]
            while True:
                tok = int(rng.integers(0, vocab))
                if tok not in sib or len(sib) >= vocab:
                    break
            tokens[b, node] = tok
    logits = rng.standard_normal((batch, t + 1, vocab), dtype=np.float32)
    paths = []
    for b in range(batch):
        path = []
        if plant:
            leaf = int(rng.integers(0, t))
            chain = [leaf]
            while parents[b, chain[-1]] >= 0:
                chain.append(int(parents[b, chain[-1]]))
            chain = chain[::-1][:int(rng.integers(0, len(chain) + 1))]
            prev_row = 0
            for node in chain:
                logits[b, prev_row, tokens[b, node]] += 20.0
                prev_row = 1 + node
            path = chain
        paths.append(path)
    return dict(name=f"accept_s{seed}", seed=seed, batch=batch, tree_nodes=t, vocab=vocab, tree_parent=parents,
                draft_tokens=tokens, logits=logits, planted=paths)
