"""GPU parity of the HIP verify path against the CPU fp64 oracle, through the C ABI.

Sizes span several 32-key tiles, split units and 128-row M tiles with ragged tails;
the workload configs run at full size.  Bitwise identities (fast path on/off,
permuted pool, repeat runs, poisoned unused rows / workspace) need no tolerance.
"""


import numpy as np
import pytest
import torch

import mla_tree_verify_mlaverify_amd as mv
from gpu_util import DEV, compare, i32, run_gpu, run_oracle, upload, verifier_for
from oracle import mla_tree_oracle as orc
from workloads import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


# --------------------------------------------------------------------------- a.1 masks

@pytest.mark.parametrize("seed", range(4))
def test_tree_masks_bit_exact(seed):
    rng = np.random.default_rng(seed)
    for t in (1, 2, 7, 8, 31, 32, 33, 63, 64, 65, 100, 128, 129, 200, 255, 256):
        trees = [synth.random_tree(rng, t), synth.chain_tree(t),
                 np.array([int(rng.integers(-1, i)) for i in range(t)], dtype=np.int32)]
        par = np.stack(trees).astype(np.int32)
        masks, err = mv.tree_masks(i32(par))
        torch.cuda.synchronize()
        got = masks.cpu().numpy().view(np.uint64)
        for b in range(len(trees)):
            assert np.array_equal(got[b], orc.ancestor_mask_words(par[b])), (t, b)
            if t <= 64:
                assert np.array_equal(got[b][:, 0], orc.ancestor_masks(par[b]))
        assert np.all(err.cpu().numpy() == 0)


def test_tree_masks_flag_bad_parents():
    par = np.array([[-1, 0, 1, 2], [-1, 0, 2, 1], [-1, 5, 0, 0], [0, -1, 1, 1], [-1, -2, 0, 0]], dtype=np.int32)
    masks, err = mv.tree_masks(i32(par))
    torch.cuda.synchronize()
    e = err.cpu().numpy()
    m = masks.cpu().numpy().view(np.uint64)[:, :, 0]
    assert e.tolist() == [0, mv.DEVERR_BAD_PARENT, mv.DEVERR_BAD_PARENT, mv.DEVERR_BAD_PARENT, mv.DEVERR_BAD_PARENT]
    assert np.array_equal(m[0], orc.ancestor_masks(par[0]))
    assert np.all(m[1:] == 0)


# --------------------------------------------------------------------------- small parity

SMALL = [
    # seed, prefix per request, T, H, tree kind, split_tokens
    (0, [0], 1, 1, "random", 0),
    (1, [1], 1, 8, "random", 0),
    (2, [31, 33], 5, 8, "random", 0),
    (3, [100, 0, 257], 8, 8, "forest", 32),
    (4, [300], 32, 8, "random", 64),
    (5, [129, 64], 33, 4, "chain", 0),
    (6, [1000], 64, 8, "random", 0),
    (7, [513, 77, 0, 1], 17, 16, "forest", 96),
    (8, [2047], 64, 3, "random", 128),
    (9, [640, 641], 64, 2, "random", 0),
    # limits: 128 heads (M = 8192 rows, 64 M tiles), one node of 128 heads, large batches
    (10, [1000], 64, 128, "random", 0),
    (11, [3000], 1, 128, "random", 0),
    (12, [64] * 300, 2, 2, "random", 0),
    (13, [5] * 1024, 1, 1, "chain", 0),
    (14, [0] * 1000 + [4097], 3, 8, "random", 0),
    # trees over 64 nodes: four mask words per row, up to 8 tree tiles in the last unit
    (15, [700], 65, 8, "random", 0),
    (16, [300, 1200], 100, 4, "forest", 256),
    (17, [1000], 128, 8, "chain", 0),
    (18, [2000], 256, 8, "random", 0),
    (19, [0, 513], 200, 2, "chain", 0),
    (20, [129], 256, 1, "forest", 64),
    # ragged prefixes that round up past one workgroup per CU: the split search
    (21, [30000] + [200] * 40, 2, 8, "random", 0),
    (22, [9000, 130, 4000, 131, 700, 129] * 4, 32, 16, "random", 0),
    # one M tile of 65..128 rows (gathers staged in VGPRs): big tree, fixed split with a tail
    (23, [900], 100, 1, "random", 0),
    (24, [1234], 16, 8, "forest", 96),
]


@pytest.mark.parametrize("seed,prefix,t,h,tree,split", SMALL)
def test_small_parity(seed, prefix, t, h, tree, split):
    cfg = synth.small_config(seed, batch=len(prefix), prefix=prefix, tree_nodes=t, heads=h,
                             slots=max(4096, 2 * (sum(prefix) + len(prefix) * t)), tree=tree, q_scale=1.0)
    out, lse, v = run_gpu(cfg, split_tokens=split)
    ref_out, ref_lse = run_oracle(cfg)
    compare(out, lse, ref_out, ref_lse)
    plan = v.read_plan()
    # the unit partition covers each prefix exactly once, in split_len pieces
    offs = orc.request_offsets(cfg["prefix_lens"], t)
    first = 0
    for b, rq in enumerate(plan["requests"]):
        assert rq["key_offset"] == offs[b] and rq["prefix_len"] == prefix[b]
        assert rq["first_unit"] == first and rq["units"] == units_of(prefix[b], plan["split_len"], 0 if split else t)
        first += rq["units"]
        assert rq["error_bits"] == 0
    assert plan["total_units"] == first
    if split:
        assert plan["split_len"] == split
    else:
        check_auto_split(prefix, t, plan["split_len"], plan["n_mtiles"])


def units_of(p, s, t):
    """Units of a request of p prefix tokens at split length s: under an automatic split its
    t tree keys (in whole 32-key tiles) count as work of the last unit, which is the only
    unit allowed past the prefix; under a fixed split (t = 0) only the prefix counts."""
    tk = -(-t // 32) * 32
    return max(1, min(-(-(p + tk) // s), -(-p // s) + 1))


def check_auto_split(prefix, t, s, n_mtiles):
    """The automatic split length is the smallest multiple of 32 (at least 128) that keeps
    the unit count within one workgroup per CU per M tile (256 CUs), when the batch allows."""
    target = -(-256 // n_mtiles)
    units = lambda x: sum(units_of(p, x, t) for p in prefix)
    work = sum(prefix) + len(prefix) * (-(-t // 32) * 32)
    floor = max(128, -(-(-(-work // target)) // 32) * 32)
    assert s % 32 == 0 and s >= floor
    if len(prefix) < target:
        assert units(s) <= target
        assert s == floor or units(s - 32) > target


# --------------------------------------------------------------------------- workload configs

@pytest.mark.parametrize("i", [0, 1, 2, 3, 4, 5, 6])
def test_config_parity_full(i):
    """Every row of every workload, element by element (the 185k and batch workloads take the
    oracle about a second each)."""
    cfg = synth.make_config(i)
    out, lse, v = run_gpu(cfg)
    plan = v.read_plan()
    check_auto_split(cfg["prefix_lens"].tolist(), cfg["tree_nodes"], plan["split_len"], plan["n_mtiles"])
    ref_out, ref_lse = run_oracle(cfg)
    print(i, compare(out, lse, ref_out, ref_lse))


def test_largest_rows_per_request():
    # 128 heads x 256 nodes = 32,768 rows per request: 256 M tiles, one unit each, four mask
    # words per row; the oracle evaluates a sample of the nodes.
    cfg = synth.small_config(31, batch=1, prefix=[300], tree_nodes=256, heads=128,
                             slots=4096, tree="random", q_scale=1.0)
    out, lse, v = run_gpu(cfg)
    plan = v.read_plan()
    assert plan["n_mtiles"] == 256 and plan["total_units"] == 1
    nodes = [(0, n) for n in (0, 1, 77, 128, 200, 255)]
    ref_out, ref_lse = run_oracle(cfg, nodes=nodes)
    compare(out, lse, ref_out, ref_lse)


# --------------------------------------------------------------------------- sensitive variants

@pytest.mark.parametrize("variant", ["sorted", "contiguous", "sharp", "needle_prefix", "needle_tree", "prefix0",
                                     "chain"])
def test_variant_parity(variant):
    cfg = synth.make_config(1, variant=variant)
    out, lse, _ = run_gpu(cfg)
    ref_out, ref_lse = run_oracle(cfg)
    compare(out, lse, ref_out, ref_lse)
    if variant.startswith("needle"):
        assert np.abs(ref_out).max() > 1.0  # the needle dominates somewhere


@pytest.mark.parametrize("variant", ["sharp", "needle_prefix", "needle_tree", "prefix0", "chain", "qzero"])
def test_variant_parity_one_m_tile(variant):
    # 64 rows in one M tile, three units; the needles raise a row's reference after its
    # first tile (a rescale of the row's accumulator and sum)
    cfg = synth.make_config(0, variant=variant)
    out, lse, _ = run_gpu(cfg)
    ref_out, ref_lse = run_oracle(cfg)
    compare(out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("seed,prefix,t,h,split", [(40, [4000], 8, 8, 160), (41, [1, 95, 300, 2000], 5, 8, 0),
                                                   (42, [700], 64, 1, 0), (43, [37, 0], 16, 4, 0)])
def test_one_m_tile_many_tiles(seed, prefix, t, h, split):
    # single-M-tile shapes with units of several tiles (odd and even counts), tree tiles,
    # and a request with no prefix
    cfg = synth.small_config(seed, batch=len(prefix), prefix=prefix, tree_nodes=t, heads=h,
                             slots=max(4096, 2 * (sum(prefix) + len(prefix) * t)), tree="random", q_scale=1.0)
    out, lse, v = run_gpu(cfg, split_tokens=split)
    ref_out, ref_lse = run_oracle(cfg)
    compare(out, lse, ref_out, ref_lse)
    assert v.read_plan()["n_mtiles"] == 1


def test_column_scales_keep_per_column_precision():
    """V columns span 2^-12 .. 2^12 (q scaled inversely, so the scores are those of the
    unscaled data).  Each output column divided by its scale must meet the bar of unscaled
    data: rounding anywhere on the path must stay relative to the column itself."""
    cfg = synth.make_config(1, variant="colscale")
    out, lse, _ = run_gpu(cfg)
    ref_out, ref_lse = run_oracle(cfg)
    s = synth.column_scales()
    print(compare(out / s, lse, ref_out / s, ref_lse))


def test_ragged_trees_by_padding():
    """Requests with 5 and 70 nodes in one call: the smaller tree is padded to 70 nodes with
    extra roots (their own tree slots); the real nodes' rows must equal the oracle's for
    the unpadded trees."""
    rng = np.random.default_rng(31)
    cfg = synth.small_config(31, batch=2, prefix=[400, 900], tree_nodes=70, heads=4, slots=8192)
    par = cfg["tree_parent"].copy()
    small = synth.random_tree(rng, 5)
    par[0, :5] = small
    par[0, 5:] = -1  # padding: extra roots, seen by nobody else
    cfg["tree_parent"] = par
    out, lse, _ = run_gpu(cfg)
    ref_out, ref_lse = run_oracle(cfg)
    # the oracle of request 0 alone, with its real 5-node tree
    seg0 = cfg["kv_indices"][:400 + 70]
    solo_idx = np.concatenate([seg0[:400], seg0[400:405]])
    solo_out, solo_lse = orc.verify_attention(cfg["q"][:5], cfg["pool"], solo_idx, np.array([400]),
                                              small[None, :], cfg["sm_scale"])
    compare(out[:5], lse[:5], solo_out, solo_lse)
    compare(out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("cfg_i,split", [(1, 256), (0, 96), (2, 0)])
def test_reference_raised_at_every_unit_end(cfg_i, split):
    """A dominant key at the last prefix key of every unit: every row's softmax reference is
    raised in the last prefix tile of each unit, where the rows' partial sums are rescaled
    once.  Matches the oracle; the plan readback counts the waves that rescaled."""
    cfg = synth.make_config(cfg_i)
    v = verifier_for(cfg, split_tokens=split)
    run_gpu(cfg, v)
    plan = v.read_plan()  # the split the automatic plan chooses (and a fresh rescale count)
    s = plan["split_len"]
    planted = synth.plant_unit_end_needles(cfg, s)
    out, lse, _ = run_gpu(planted, v)
    plan = v.read_plan()
    assert plan["split_len"] == s
    prefix_units = sum(min(r["units"], -(-r["prefix_len"] // s)) for r in plan["requests"])
    waves = -(-cfg["heads"] * cfg["tree_nodes"] // 32)  # waves holding rows, over all M tiles
    assert plan["rescales"] >= prefix_units - 1 and plan["rescales"] <= prefix_units * waves, plan["rescales"]
    ref_out, ref_lse = run_oracle(planted)
    assert np.abs(ref_out).max() > 1.0  # the needles dominate
    print(compare(out, lse, ref_out, ref_lse))


def test_q_zero_lse_is_log_count():
    cfg = synth.make_config(0, variant="qzero")
    out, lse, _ = run_gpu(cfg)
    g = [257, 258, 259, 260, 258, 259, 259, 260]
    np.testing.assert_allclose(lse, np.log(np.array(g, dtype=np.float64))[:, None].repeat(8, 1), atol=2e-6)
    ref_out, ref_lse = run_oracle(cfg)
    compare(out, lse, ref_out, ref_lse)


def test_row_stride_larger_than_row():
    cfg = synth.small_config(21, batch=2, prefix=[300, 45], tree_nodes=9, heads=8, slots=2048, row_stride=640)
    out, lse, _ = run_gpu(cfg)
    ref_out, ref_lse = run_oracle(cfg)
    compare(out, lse, ref_out, ref_lse)  # the NaN padding columns are never read


# --------------------------------------------------------------------------- bitwise identities

def test_fast_path_is_bit_identical():
    cfg = synth.make_config(1, variant="contiguous")
    a, la, v = run_gpu(cfg)
    assert v.read_plan()["fast_units"] > 0
    b, lb, v = run_gpu(cfg, flags=mv.FLAG_NO_FASTPATH)
    assert v.read_plan()["fast_units"] == 0
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def prefix_units(plan):
    """Units that hold prefix keys (a request's units all do, except a last one past its prefix)."""
    n = 0
    for rq in plan["requests"]:
        s = plan["split_len"]
        n += min(rq["units"], -(-rq["prefix_len"] // s))
    return n


@pytest.mark.parametrize("variant", ["contiguous", "sorted"])
def test_fast_path_on_long_units(variant):
    """The 65k workload with its indices defragmented into one run, or only sorted: units of
    about a thousand keys, so the run check also takes its rounds past the first 256 keys.
    Each unit of the run takes the fast path; sorted indices (gaps between slots) take none.
    Both match the oracle and are bit-identical to the row-by-row gathers."""
    cfg = synth.make_config(2, variant=variant)
    out, lse, v = run_gpu(cfg)
    plan = v.read_plan()
    assert plan["split_len"] > 256
    expect = prefix_units(plan) if variant == "contiguous" else 0
    assert plan["fast_units"] == expect, (plan["fast_units"], expect)
    ref_out, ref_lse = run_oracle(cfg)
    print(variant, compare(out, lse, ref_out, ref_lse))
    b, lb, v2 = run_gpu(cfg, flags=mv.FLAG_NO_FASTPATH)
    assert v2.read_plan()["fast_units"] == 0
    assert np.array_equal(out, b) and np.array_equal(lse, lb)


@pytest.mark.parametrize("split", [1024, 0])
def test_fast_path_rejects_broken_runs(split):
    """A contiguous prefix with single slots replaced by a slot outside the run, at unit key
    100 (the check's first round), 300 and 700 (later rounds), a unit's last key, and the
    request's last prefix key.  Exactly the units holding a break leave the fast path; the
    output matches the oracle and the row-by-row gathers bit for bit."""
    prefix, t = 20517, 64  # 512 rows: the automatic split is then longer than 256 keys
    cfg = synth.small_config(50, batch=1, prefix=[prefix], tree_nodes=t, heads=8, slots=65536, tree="random",
                             q_scale=1.0)
    cfg = synth.apply_variant(cfg, "contiguous")
    v0 = verifier_for(cfg, split_tokens=split)
    run_gpu(cfg, v0)
    plan = v0.read_plan()
    s = plan["split_len"]
    assert s > 256 and plan["fast_units"] == prefix_units(plan)
    last = (prefix - 1) // s  # the last unit holding prefix keys
    base = int(cfg["kv_indices"][0])
    assert base >= 8 and last > 5, "free slots below the run, and enough units"
    breaks = {1: 100, 2: 300, 4: s - 1, 5: min(700, s - 2), last: prefix - 1 - last * s}
    broken = dict(cfg)
    idx = cfg["kv_indices"].copy()
    for j, (u, k) in enumerate(sorted(breaks.items())):
        assert 0 <= k < s and u * s + k < prefix
        idx[u * s + k] = base - 1 - j  # a free slot below the run (its row is ordinary data)
    broken["kv_indices"] = idx
    out, lse, v = run_gpu(broken, split_tokens=split)
    plan = v.read_plan()
    assert plan["split_len"] == s
    assert plan["fast_units"] == prefix_units(plan) - len(breaks), plan
    ref_out, ref_lse = run_oracle(broken)
    compare(out, lse, ref_out, ref_lse)
    b, lb, _ = run_gpu(broken, split_tokens=split, flags=mv.FLAG_NO_FASTPATH)
    assert np.array_equal(out, b) and np.array_equal(lse, lb)


def test_permuted_pool_is_bit_identical():
    cfg = synth.make_config(1)
    perm = synth.permute_pool(cfg, np.random.default_rng(7))
    a, la, _ = run_gpu(cfg)
    b, lb, _ = run_gpu(perm)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_repeat_runs_are_bit_identical():
    cfg = synth.make_config(2)
    d = upload(cfg)
    v = verifier_for(cfg)
    a, la, _ = run_gpu(cfg, v, d)
    b, lb, _ = run_gpu(cfg, v, d)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_poisoned_unused_rows_do_not_change_output():
    cfg = synth.make_config(1)
    a, la, _ = run_gpu(cfg)
    b, lb, _ = run_gpu(synth.apply_variant(cfg, "poison_unused"))
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_poisoned_workspace_does_not_change_output():
    cfg = synth.small_config(22, batch=3, prefix=[700, 5, 1500], tree_nodes=24, heads=8, slots=8192)
    d = upload(cfg)
    v = verifier_for(cfg)
    a, la, _ = run_gpu(cfg, v, d)
    v.workspace.fill_(0xFF)  # NaN in every float of the workspace
    torch.cuda.synchronize()
    b, lb, _ = run_gpu(cfg, v, d)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


@pytest.mark.parametrize("split", [32, 64, 256, 1024, 4096])
def test_split_length_changes_only_rounding(split):
    cfg = synth.make_config(1)
    out, lse, v = run_gpu(cfg, split_tokens=split)
    assert v.read_plan()["split_len"] == split
    ref_out, ref_lse = run_oracle(cfg)
    compare(out, lse, ref_out, ref_lse)


# --------------------------------------------------------------------------- errors

# 12 nodes x H heads: 48 rows (helper waves gather every tile), 96 rows (register-staged
# gathers) or 192 rows (two M tiles, LDS-DMA gathers); the bad parent ends the workgroup after
# the tree check on each path
@pytest.mark.parametrize("heads", [4, 8, 16])
def test_device_errors_poison_only_the_offending_request(heads):
    cfg = synth.small_config(30, batch=4, prefix=[200, 300, 100, 50], tree_nodes=12, heads=heads, slots=4096)
    bad = dict(cfg)
    par = cfg["tree_parent"].copy()
    par[1, 5] = 7  # parent after the node
    idx = cfg["kv_indices"].copy()
    idx[200 + 12 + 300 + 12 + 17] = 4096 + 3  # request 2, prefix slot 17: outside the pool
    plens = cfg["prefix_lens"].copy()
    bad.update(tree_parent=par, kv_indices=idx)
    v = verifier_for(cfg, max_prefix=300)
    out, lse, _ = run_gpu(bad, v)
    flags = v.read_device_errors()
    assert flags == mv.DEVERR_BAD_PARENT | mv.DEVERR_BAD_INDEX
    assert v.read_device_errors() == 0  # read clears
    t = 12
    ref_out, ref_lse = run_oracle(cfg)
    for b in range(4):
        rows = slice(b * t, (b + 1) * t)
        if b in (1, 2):
            assert np.all(np.isnan(out[rows])) and np.all(np.isnan(lse[rows]))
        else:
            compare(out[rows], lse[rows], ref_out[rows], ref_lse[rows])
    # prefix longer than max_prefix_len
    plens[3] = 301
    bad2 = synth.small_config(30, batch=4, prefix=list(plens), tree_nodes=12, heads=heads, slots=4096)
    out2, lse2, _ = run_gpu(bad2, v)
    assert v.read_device_errors() == mv.DEVERR_BAD_PREFIX
    assert np.all(np.isnan(out2[3 * t:])) and np.all(np.isfinite(out2[:3 * t]))


def test_host_argument_errors_enqueue_nothing():
    cfg = synth.make_config(0)
    v = verifier_for(cfg)
    d = upload(cfg)
    out = torch.full((8, 8, 512), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((8, 8), 7.0, dtype=torch.float32, device=DEV)
    lib = v.lib
    import ctypes
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [d["q"].data_ptr(), d["pool"].data_ptr(), d["kv_indices"].data_ptr(), d["prefix_lens"].data_ptr(),
            d["tree_parent"].data_ptr(), out.data_ptr(), lse.data_ptr(), s]
    assert lib.mlaverify_run(v.handle, 2, 8, *args) == mv.binding.ERR_INVALID_ARG  # batch > max_batch
    assert lib.mlaverify_run(v.handle, 1, 9, *args) == mv.binding.ERR_INVALID_ARG  # T > max_tree_nodes
    bad = list(args)
    bad[0] = d["q"].data_ptr() + 2  # misaligned q
    assert lib.mlaverify_run(v.handle, 1, 8, *bad) == mv.binding.ERR_INVALID_ARG
    bad = list(args)
    bad[5] = 0
    assert lib.mlaverify_run(v.handle, 1, 8, *bad) == mv.binding.ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(out.float() == 7.0) and torch.all(lse == 7.0)
