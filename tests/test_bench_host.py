"""Host logic of bench.py, pinned on the CPU: the algorithmic bytes and flops behind every
reported rate and roofline fraction, the tie between stored profiler counters and the
kernel sources, and the single-GPU guard."""

import os
import subprocess
import sys

import numpy as np

import bench
from workloads import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def visible_counts(parents, prefix):
    """Keys each node sees, by walking its ancestor chain (the node itself included)."""
    out = []
    for i in range(len(parents)):
        n, j = 0, i
        while j >= 0:
            n += 1
            j = parents[j]
        out.append(prefix + n)
    return out


def test_tiny_counts_by_hand():
    # 1 request, 256-token prefix, tree [-1,0,1,2,0,4,1,6]: visible keys 257..260 per node
    cfg = synth.make_config(0)
    c = bench.algorithmic_counts(cfg)
    assert visible_counts(list(cfg["tree_parent"][0]), 256) == [257, 258, 259, 260, 258, 259, 259, 260]
    assert c["keys"] == 264
    assert c["kv_bytes"] == 264 * 1152
    assert c["flops"] == 2 * 8 * 2070 * 1088  # 2 flops x heads x visible keys x (576 + 512)
    assert c["total_bytes"] == 264 * 1152 + 264 * 4 + 8 * 8 * 576 * 2 + 8 * 8 * (512 * 2 + 4)


def test_counts_match_ancestor_walk_on_random_batches():
    rng = np.random.default_rng(11)
    for _ in range(5):
        b, t, h = int(rng.integers(1, 5)), int(rng.integers(1, 40)), int(rng.integers(1, 17))
        prefix = [int(x) for x in rng.integers(0, 3000, b)]
        cfg = synth.small_config(int(rng.integers(0, 1 << 30)), batch=b, prefix=prefix, tree_nodes=t, heads=h,
                                 slots=2 * (sum(prefix) + b * t) + 8)
        c = bench.algorithmic_counts(cfg)
        vis = sum(sum(visible_counts(list(cfg["tree_parent"][k]), prefix[k])) for k in range(b))
        assert c["flops"] == 2 * h * vis * 1088
        assert c["keys"] == sum(prefix) + b * t
        assert c["prefix_flops"] == 2 * h * t * sum(prefix) * 1088


def test_source_hash_ignores_comments_only():
    src = 'int a = 1;  // the count\n/* block\n comment */ asm("s_nop 1 // kept");\nchar c = \'"\';\n'
    same = 'int a = 1;\n// another comment\nasm("s_nop 1 // kept");   char c = \'"\';'
    assert bench.code_text(src) == bench.code_text(same)
    assert bench.code_text(src) != bench.code_text(src.replace("1;", "2;"))
    assert bench.code_text(src) != bench.code_text(src.replace("s_nop 1 // kept", "s_nop 2 // kept"))


def test_stored_traffic_follows_the_kernel_sources():
    # the committed counters are reported only for the sources they were taken from
    path = os.path.join(ROOT, "profiles", "k_partial_p185000_t64_h8.md")
    text = open(path).read()
    recorded = text.split('"source_sha256_16": "')[1].split('"')[0]
    got = bench.stored_traffic("p185000_t64_h8")
    if recorded == bench.source_hash():
        assert got is not None and got > 213_000_000  # at least the KV rows of one launch
    else:
        assert got is None
    assert bench.stored_traffic("no_such_workload") is None
    f = bench.profile_fields("p185000_t64_h8")
    if recorded == bench.source_hash():
        assert 0.0 < f["l2_hit_rate"] < 1.0 and f["occupancy"]["waves_per_simd"] >= 1
    else:
        assert f["l2_hit_rate"] is None and f["occupancy"] is None
    assert bench.profile_fields("no_such_workload") == {"l2_hit_rate": None, "occupancy": None, "profile": None}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_every_package_name_the_bench_calls_exists():
    # the bench reaches the library only through the package: each `mv.<name>` it uses must be
    # exported (a missing one would only show on the GPU, in the middle of the default run)
    import re

    import mla_tree_verify_mlaverify_amd as mv

    names = set(re.findall(r"\bmv\.([A-Za-z_]\w*)", open(os.path.join(ROOT, "bench.py")).read()))
    assert names and "probe_gather" in names
    missing = sorted(n for n in names if not hasattr(mv, n))
    assert not missing, missing


def test_ragged_workload_is_a_truncation_of_the_batch():
    cfg, rag = bench.ragged_workload()
    B, T, H = cfg["batch"], cfg["tree_nodes"], cfg["heads"]
    tl = rag["tree_lens"]
    assert tl[0] == T and tl.min() >= 4 and tl.max() <= T
    assert rag["q"].shape == (int(tl.sum()), H, 576)
    offs = synth.request_offsets(cfg["prefix_lens"], T)
    o, r = 0, 0
    for b in range(B):
        p, t = int(cfg["prefix_lens"][b]), int(tl[b])
        # the request's prefix entries and its first t tree entries, in order
        assert np.array_equal(rag["kv_indices"][o: o + p + t], cfg["kv_indices"][offs[b]: offs[b] + p + t])
        par = rag["tree_parent"][r: r + t]
        assert np.array_equal(par, cfg["tree_parent"][b, :t])
        assert all(-1 <= par[i] < i for i in range(t))
        assert np.array_equal(rag["q"][r: r + t], cfg["q"].reshape(B, T, H, 576)[b, :t])
        o += p + t
        r += t
    assert o == len(rag["kv_indices"])


def test_ragged_counts_equal_the_padded_counts_at_full_trees():
    # with every request at the full tree, the ragged call is the padded one: same keys, flops
    cfg, _ = bench.ragged_workload()
    B, T = cfg["batch"], cfg["tree_nodes"]
    full = dict(prefix_lens=cfg["prefix_lens"].astype(np.int32), tree_lens=np.full(B, T, np.int32),
                tree_parent=cfg["tree_parent"].reshape(-1))
    rc, pc = bench.ragged_counts(cfg, full), bench.algorithmic_counts(cfg)
    assert rc["flops"] == pc["flops"] and rc["kv_bytes"] == pc["kv_bytes"]
    assert rc["total_bytes"] == pc["total_bytes"]
    # and one node fewer in request 0 removes exactly that node's visible keys
    less = dict(full, tree_lens=np.array([T - 1] + [T] * (B - 1), np.int32),
                tree_parent=np.concatenate([cfg["tree_parent"][0, : T - 1], cfg["tree_parent"][1:].reshape(-1)]))
    seen = visible_counts(list(cfg["tree_parent"][0]), int(cfg["prefix_lens"][0]))[T - 1]
    assert pc["flops"] - bench.ragged_counts(cfg, less)["flops"] == 2 * cfg["heads"] * seen * 1088
