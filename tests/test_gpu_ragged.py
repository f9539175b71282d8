"""GPU parity of the ragged verify pass (mlaverify_run_ragged: a tree size per request, rows
packed request after request) against the CPU fp64 oracle's ragged definition, through the
C ABI.  Every request is drawn on its own from the workload recipe and the batch is packed
(rows, parents, index segments), with all requests reading one shared pool."""

import numpy as np
import pytest
import torch

import mla_tree_verify_mlaverify_amd as mv
from gpu_util import DEV, bf16, compare, i32
from oracle import mla_tree_oracle as orc
from workloads import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def ragged_case(seed, prefix, tree_lens, heads, slots, q_scale=1.0):
    parts = [synth.small_config(seed + 7 * b, batch=1, prefix=[p], tree_nodes=t, heads=heads, slots=slots,
                                tree="forest" if b % 3 == 2 else "random", q_scale=q_scale)
             for b, (p, t) in enumerate(zip(prefix, tree_lens))]
    return dict(q=np.concatenate([c["q"] for c in parts]), pool=parts[0]["pool"],
                kv_indices=np.concatenate([c["kv_indices"] for c in parts]).astype(np.int32),
                prefix_lens=np.array(prefix, dtype=np.int32), tree_lens=np.array(tree_lens, dtype=np.int32),
                tree_parent=np.concatenate([c["tree_parent"][0] for c in parts]).astype(np.int32),
                heads=heads, slots=slots, sm_scale=parts[0]["sm_scale"])


def run_ragged(case, max_t=None, split=0, v=None, out_fill=None, page_size=0):
    max_t = max_t or int(case["tree_lens"].max())
    v = v or mv.Verifier(num_heads=case["heads"], max_batch=len(case["prefix_lens"]), max_tree_nodes=max_t,
                         max_prefix_len=max(1, int(case["prefix_lens"].max())), pool_slots=case["slots"],
                         sm_scale=case["sm_scale"], split_tokens=split, page_size=page_size, device=DEV)
    rows = case["q"].shape[0]
    out = torch.full((rows, case["heads"], 512), out_fill if out_fill is not None else float("nan"),
                     dtype=torch.bfloat16, device=DEV)
    lse = torch.full((rows, case["heads"]), out_fill if out_fill is not None else float("nan"), dtype=torch.float32,
                     device=DEV)
    v.run_ragged(bf16(case["q"]), bf16(case["pool"]), i32(case["kv_indices"]), i32(case["prefix_lens"]),
                 i32(case["tree_lens"]), i32(case["tree_parent"]), max_t, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), v


def oracle(case):
    return orc.verify_attention_ragged(case["q"], case["pool"], case["kv_indices"], case["prefix_lens"],
                                       case["tree_lens"], case["tree_parent"], case["sm_scale"])


def expected_ragged_plan(prefix, tree_lens, heads, split):
    """The split and units the ragged plan must choose (at most 64 requests): request b fills
    mt_b = ceil(H T_b / 128) M tiles and each of its units takes mt_b workgroups; under an
    automatic split the length is the smallest multiple of 32, at least 128 and at least
    ceil(sum_b mt_b (P_b + tkeys_b) / budget), whose weighted unit count fits the budget of
    ceil(256 / M tiles) x M tiles workgroups (when the batch allows)."""
    cdiv = lambda x, y: -(-x // y)
    n_mt = cdiv(heads * max(tree_lens), 128)
    budget = cdiv(256, n_mt) * n_mt
    mt = [max(1, cdiv(heads * t, 128)) for t in tree_lens]
    tk = [0 if split else cdiv(t, 32) * 32 for t in tree_lens]
    units_at = lambda s: [max(1, min(cdiv(p + k, s), cdiv(p, s) + 1)) for p, k in zip(prefix, tk)]
    items_at = lambda s: sum(u * m for u, m in zip(units_at(s), mt))
    if split:
        return split, units_at(split)
    work = sum((p + k) * m for p, k, m in zip(prefix, tk, mt))
    s = max(128, cdiv(cdiv(work, budget), 32) * 32)
    if items_at(s) > budget and sum(mt) < budget:
        s += 32
        while items_at(s) > budget:
            s += 32
    return s, units_at(s)


def check_ragged_plan(v, case, split):
    s, units = expected_ragged_plan([int(p) for p in case["prefix_lens"]], [int(t) for t in case["tree_lens"]],
                                    case["heads"], split)
    plan = v.read_plan()
    assert plan["split_len"] == s
    assert [r["units"] for r in plan["requests"]] == units
    assert [r["first_unit"] for r in plan["requests"]] == list(np.cumsum([0] + units[:-1]))
    assert plan["total_units"] == sum(units)


@pytest.mark.parametrize("seed,prefix,tree_lens,heads,split", [
    (80, [3000, 1, 700, 4096], [1, 5, 64, 200], 8, 0),     # big-tree launch (max 200): four mask words
    (81, [1500, 0, 257, 33, 9000], [64, 5, 1, 17, 33], 8, 0),
    (82, [1500, 0, 257, 33, 9000], [64, 5, 1, 17, 33], 8, 256),
    (83, [4000, 100, 2000], [8, 1, 3], 8, 0),                # one M tile: the helper-wave gathers
    (84, [640] * 6, [2, 31, 32, 33, 63, 64], 16, 0),         # tile and M-tile edges
    (85, [2500, 40, 900], [16, 3, 9], 8, 0),                 # one M tile of 128 rows: register-staged gathers
])
def test_ragged_parity(seed, prefix, tree_lens, heads, split):
    case = ragged_case(seed, prefix, tree_lens, heads, slots=max(4096, 2 * (sum(prefix) + sum(tree_lens))))
    out, lse, v = run_ragged(case, split=split)
    assert v.read_device_errors() == 0
    ref_out, ref_lse = oracle(case)
    print(compare(out, lse, ref_out, ref_lse))
    check_ragged_plan(v, case, split)


@pytest.mark.parametrize("seed", range(6))
def test_ragged_random_shapes(seed):
    # random batches: heads, tree sizes (1 to 2 M tiles and past 64 nodes), prefixes and the
    # split vary, against the oracle and the plan's host model
    rng = np.random.default_rng(500 + seed)
    b = int(rng.integers(2, 13))
    heads = int(rng.choice([2, 4, 8, 16]))
    tree_lens = [int(x) for x in rng.integers(1, 81, size=b)]
    prefix = [int(x) for x in rng.integers(0, 3000, size=b)]
    split = int(rng.choice([0, 0, 96, 512]))
    case = ragged_case(500 + seed, prefix, tree_lens, heads, slots=max(4096, 2 * (sum(prefix) + sum(tree_lens))))
    out, lse, v = run_ragged(case, split=split)
    assert v.read_device_errors() == 0
    ref_out, ref_lse = oracle(case)
    compare(out, lse, ref_out, ref_lse)
    check_ragged_plan(v, case, split)


def test_ragged_bench_workload_full_size():
    # the ragged batch bench.py times (8 requests, 1k-131k prefixes, trees of 4-32 nodes, 16
    # heads), every row against the oracle, in the launch configuration of the bench
    import bench

    cfg, rag = bench.ragged_workload()
    case = dict(q=rag["q"], pool=cfg["pool"], kv_indices=rag["kv_indices"], prefix_lens=rag["prefix_lens"],
                tree_lens=rag["tree_lens"], tree_parent=rag["tree_parent"], heads=cfg["heads"],
                slots=cfg["slots"], sm_scale=cfg["sm_scale"])
    v = mv.Verifier(num_heads=cfg["heads"], max_batch=cfg["batch"], max_tree_nodes=cfg["tree_nodes"],
                    max_prefix_len=int(cfg["prefix_lens"].max()), pool_slots=cfg["slots"],
                    sm_scale=cfg["sm_scale"], device=DEV)
    out, lse, v = run_ragged(case, max_t=cfg["tree_nodes"], v=v)
    assert v.read_device_errors() == 0
    check_ragged_plan(v, case, 0)
    ref_out, ref_lse = oracle(case)
    print(compare(out, lse, ref_out, ref_lse))


def test_ragged_batch_over_64_requests():
    # more than 64 requests take the workgroup plan, which plans as if every tree were the
    # largest (partial rows apart at first_unit * M), with a tree size per request
    rng = np.random.default_rng(88)
    prefix = [int(x) for x in rng.integers(0, 400, size=70)]
    tree_lens = [int(x) for x in rng.integers(1, 13, size=70)]
    tree_lens[5] = 12
    case = ragged_case(88, prefix, tree_lens, 4, slots=max(4096, 2 * (sum(prefix) + sum(tree_lens))))
    out, lse, v = run_ragged(case)
    assert v.read_device_errors() == 0
    ref_out, ref_lse = oracle(case)
    compare(out, lse, ref_out, ref_lse)
    plan = v.read_plan()
    assert [r["first_unit"] for r in plan["requests"]] == list(np.cumsum([0] + [r["units"] for r in plan["requests"]][:-1]))


def test_ragged_with_equal_trees_is_run_bit_for_bit():
    cfg = synth.small_config(85, batch=3, prefix=[1000, 20, 333], tree_nodes=24, heads=8, slots=8192, q_scale=1.0)
    case = dict(q=cfg["q"], pool=cfg["pool"], kv_indices=cfg["kv_indices"], prefix_lens=cfg["prefix_lens"],
                tree_lens=np.full(3, 24, dtype=np.int32), tree_parent=cfg["tree_parent"].reshape(-1),
                heads=8, slots=8192, sm_scale=cfg["sm_scale"])
    out, lse, v = run_ragged(case)
    o2, l2 = v.run(bf16(cfg["q"]), bf16(cfg["pool"]), i32(cfg["kv_indices"]), i32(cfg["prefix_lens"]),
                   i32(cfg["tree_parent"]))
    torch.cuda.synchronize()
    assert np.array_equal(out, o2.float().cpu().numpy()) and np.array_equal(lse, l2.cpu().numpy())


def test_ragged_below_the_launch_maximum():
    # max_T of the call (96, a big-tree launch) above every request's tree
    case = ragged_case(86, [500, 1200], [7, 40], 4, slots=4096)
    out, lse, _ = run_ragged(case, max_t=96)
    ref_out, ref_lse = oracle(case)
    compare(out, lse, ref_out, ref_lse)


def test_bad_tree_length_poisons_that_request_and_later_ones():
    case = ragged_case(87, [300, 400, 500], [4, 6, 5], 8, slots=4096)
    bad = dict(case, tree_lens=np.array([4, 9, 5], dtype=np.int32))  # 9 > max_T = 6
    out, lse, v = run_ragged(bad, max_t=6, out_fill=7.0)
    assert v.read_device_errors() == mv.DEVERR_BAD_TREE_LEN
    ref_out, ref_lse = orc.verify_attention_ragged(case["q"][:4], case["pool"], case["kv_indices"][:304],
                                                   case["prefix_lens"][:1], [4], case["tree_parent"][:4],
                                                   case["sm_scale"])
    compare(out[:4], lse[:4], ref_out, ref_lse)  # the request before the bad one is whole
    assert np.all(out[4:] == 7.0) and np.all(lse[4:] == 7.0)  # no row of the later ones is written
    zero = dict(case, tree_lens=np.array([4, 0, 5], dtype=np.int32))
    out, lse, v = run_ragged(zero, max_t=6, out_fill=7.0)
    assert v.read_device_errors() == mv.DEVERR_BAD_TREE_LEN
    compare(out[:4], lse[:4], ref_out, ref_lse)
    assert np.all(out[4:] == 7.0) and np.all(lse[4:] == 7.0)


def paged_ragged_case(seed, prefix, tree_lens, heads, slots, page):
    """The ragged case with its prefixes paged: per request the page ids of its ceil(P_b / page)
    prefix pages (distinct, below the top quarter of the pool), then its T_b tree slots (top
    quarter); returned with the same batch addressed one slot per token."""
    case = ragged_case(seed, prefix, tree_lens, heads, slots)
    rng = np.random.default_rng(40_000 + seed)
    top = slots - slots // 4
    n_pages = [-(-p // page) for p in prefix]
    pages = rng.choice(top // page, size=sum(n_pages), replace=False)
    tree = top + rng.choice(slots - top, size=sum(tree_lens), replace=False)
    segs, flat, pp, tp = [], [], 0, 0
    for p, t, n in zip(prefix, tree_lens, n_pages):
        pg, ts = pages[pp:pp + n], tree[tp:tp + t]
        pos = np.arange(p)
        segs += [pg, ts]
        flat += [pg[pos // page] * page + pos % page, ts]
        pp, tp = pp + n, tp + t
    paged = dict(case, kv_indices=np.concatenate(segs).astype(np.int32))
    per_token = dict(case, kv_indices=np.concatenate(flat).astype(np.int32))
    return paged, per_token


@pytest.mark.parametrize("seed,prefix,tree_lens,heads,page", [
    (90, [700, 0, 2100, 33], [5, 1, 40, 64], 8, 16),   # four M tiles (LDS-DMA gathers)
    (91, [1300, 257], [9, 3], 8, 64),                    # one M tile of 72 rows (register-staged)
    (92, [900, 65, 400], [2, 8, 5], 4, 8),               # one M tile of 32 rows (helper waves)
])
def test_ragged_paged_equals_its_expansion_and_oracle(seed, prefix, tree_lens, heads, page):
    paged, flat = paged_ragged_case(seed, prefix, tree_lens, heads, slots=16384, page=page)
    a, la, v = run_ragged(paged, page_size=page)
    assert v.read_device_errors() == 0
    b, lb, _ = run_ragged(flat)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    ref_out, ref_lse = oracle(flat)
    print(compare(a, la, ref_out, ref_lse))


@pytest.mark.parametrize("seed", range(4))
def test_ragged_random_paged(seed):
    # random ragged batches on paged prefixes: bit-identical to the per-token expansion (same
    # plan) and matched against the oracle
    rng = np.random.default_rng(600 + seed)
    b = int(rng.integers(2, 9))
    heads = int(rng.choice([4, 8, 16]))
    tree_lens = [int(x) for x in rng.integers(1, 70, size=b)]
    prefix = [int(x) for x in rng.integers(0, 2500, size=b)]
    page = int(rng.choice([16, 64, 256]))
    paged, flat = paged_ragged_case(600 + seed, prefix, tree_lens, heads, slots=32768, page=page)
    a, la, v = run_ragged(paged, page_size=page)
    assert v.read_device_errors() == 0
    check_ragged_plan(v, paged, 0)
    b_, lb, _ = run_ragged(flat)
    assert np.array_equal(a, b_) and np.array_equal(la, lb)
    ref_out, ref_lse = oracle(flat)
    compare(a, la, ref_out, ref_lse)
