"""Benchmark of DDTree MLA tree-verify attention on one MI355X.

One step = one full verify pass (plan + split-KV partials + LSE merge) over the
workload, with its inputs resident in HBM and the caches flushed before each call
(a 1 GiB read-modify-write), since a long-context KV does not stay cached between
decode steps.  Prints one JSON line: µs per call, KV GB/s, the partial
kernel's roofline and, unless --no-cpu, the CPU oracle timed on the host.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 3] [--warm] [--no-cpu]

Before the W warmup steps of each workload, the bench runs untimed calls for 0.3 s so that
the GPU clocks have ramped up (`settle`).  The default run times the 185k-token workload (the
headline line) and then, with the same
protocol, every other seeded workload (`per_config`), the measured stream bandwidth of the
1 GiB flush kernel (`hbm_stream_gbs`, so that %HBM is also given against it), the
scattered-read probe on the headline's rows (`gather_probe_gbs`) and the ragged batch against
the same batch padded (`ragged`, as with --op ragged).

With --op relocate it measures Tier-1 relocation instead: one call moves a 185,000-row
prefix, scattered over the lower half of a 524,288-slot pool, into one run in the upper
half (the index list is restored before each call, outside the timed region).  With
--op accept it measures greedy acceptance of a 64-node tree over fp32 logits of a
131,072-token vocabulary.  With --op gather it runs the scattered-row read probe alone: the
185k workload's prefix rows read into registers and into LDS at 256-2,048 workgroups.  With
--op ragged it times a ragged call (a tree size per request, 4-32 nodes, on the batch of 8)
against the same batch padded to its largest tree.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verify-attn \u00b5s/call + KV GB/s (% HBM peak), 64-node tree, 4k\u2013185k prefix"
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
KV_ROW_BYTES = 576 * 2
INDEX_BYTES = 4


def algorithmic_counts(cfg: dict) -> dict:
    """Bytes and flops the verify pass must move / perform, independent of the implementation."""
    from workloads import synth

    b, t, h = cfg["batch"], cfg["tree_nodes"], cfg["heads"]
    plens = cfg["prefix_lens"].astype(np.int64)
    keys = int(plens.sum()) + b * t
    kv_bytes = keys * KV_ROW_BYTES
    q_bytes = b * t * h * 576 * 2
    out_bytes = b * t * h * (512 * 2 + 4)
    total_bytes = kv_bytes + len(cfg["kv_indices"]) * INDEX_BYTES + q_bytes + out_bytes  # one entry per page when paged
    visible = 0  # sum over (request, node) of |prefix| + |ancestors incl. self|
    for bb in range(b):
        depth = synth.tree_depths(cfg["tree_parent"][bb])
        visible += t * int(plens[bb]) + int((depth + 1).sum())
    flops = 2 * h * visible * (576 + 512)
    return dict(keys=keys, kv_bytes=kv_bytes, total_bytes=total_bytes, flops=flops,
                prefix_flops=2 * h * t * int(plens.sum()) * (576 + 512))


def code_text(src: str) -> str:
    """C++ source with its comments and whitespace removed (string literals kept), so that an
    edit of the comments alone does not count as a change of the code."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c == '"' or c == "'":  # a literal, copied whole
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif c.isspace():
            i += 1
        else:
            out.append(c)
            i += 1
    return "".join(out)


def source_hash() -> str:
    """Short hash of the partial kernel's sources (code only, see code_text), to tie stored
    profiler counters to this build."""
    h = hashlib.sha256()
    for f in ("kernels.hip", "mlv_internal.h"):
        with open(os.path.join(ROOT, "mla_tree_verify_mlaverify_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def stored_profile(workload: str):
    """The committed rocprofv3 summary of k_partial on this workload (HBM bytes per launch,
    L2 hit rate, occupancy), or None when there is none or the kernel sources changed since
    the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"k_partial_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        m = re.search(r"<!-- traffic: (\{.*\}) -->", fh.read())
    if not m:
        return None
    tr = json.loads(m.group(1))
    return tr if tr.get("source_sha256_16") == source_hash() else None


def stored_traffic(workload: str):
    """HBM bytes per k_partial launch from the committed FETCH_SIZE/WRITE_SIZE counters of this
    workload (see stored_profile), or None."""
    tr = stored_profile(workload)
    return tr["bytes_per_launch"] if tr else None


def profile_fields(workload: str) -> dict:
    """L2 hit rate and occupancy of k_partial on this workload from its committed summary
    (null when absent or stale)."""
    tr = stored_profile(workload) or {}
    occ = {k: tr[k] for k in ("waves_per_simd", "workgroups_per_cu", "vgprs", "lds_bytes") if k in tr}
    return {"l2_hit_rate": tr.get("l2_hit_rate"), "occupancy": occ or None,
            "profile": f"profiles/k_partial_{workload}.md" if tr else None}


def lscpu_model() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return "unknown"


def cpu_baseline(cfg: dict, counts: dict, budget_s: float) -> dict:
    """The CPU fp64 oracle, as it stands, on the same workload (a bounded sample of its rows)."""
    from oracle import mla_tree_oracle as orc

    if cfg.get("page_size", 1) > 1:  # the oracle reads one slot per token
        cfg = dict(cfg, kv_indices=orc.expand_block_table(cfg["kv_indices"], cfg["prefix_lens"], cfg["tree_nodes"],
                                                          cfg["page_size"]))
    try:
        from threadpoolctl import threadpool_info

        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=os.cpu_count())
    except Exception:
        threads = os.cpu_count()
    t_nodes = cfg["tree_nodes"]
    all_nodes = [(bb, i) for bb in range(cfg["batch"]) for i in range(t_nodes)]
    # time one node first, then size the sample to the budget: a subset of the rows, or whole
    # calls repeated when one call is shorter than the budget
    t0 = time.perf_counter()
    orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"], cfg["tree_parent"],
                         cfg["sm_scale"], nodes=[(0, 0)])
    one = time.perf_counter() - t0
    n_nodes = int(max(1, min(len(all_nodes), budget_s / max(one, 1e-3))))
    nodes = all_nodes[:n_nodes]
    reps, secs = 0, 0.0
    t0 = time.perf_counter()
    while True:
        orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"], cfg["tree_parent"],
                             cfg["sm_scale"], nodes=nodes if len(nodes) < len(all_nodes) else None)
        reps += 1
        secs = time.perf_counter() - t0
        if len(nodes) < len(all_nodes) or secs >= 0.6 * budget_s:
            break
    frac = len(nodes) / len(all_nodes)
    est_call_s = secs / reps / frac
    what = (f"{len(nodes)} of {len(all_nodes)} tree nodes (all heads) of the same workload, {secs:.1f} s; per-call time "
            f"scaled by the node fraction" if frac < 1 else
            f"the whole call (all {len(all_nodes)} tree nodes, all heads), repeated {reps} times in {secs:.1f} s")
    return {"value": round(counts["kv_bytes"] / est_call_s / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "sample": f"{what} ({est_call_s:.2f} s/call)",
            "cpu_model": lscpu_model()}


RELOC_SLOTS, RELOC_PREFIX, RELOC_T = 524288, 185000, 64
RELOC_METRIC = "Tier-1 relocation GB/s (rows read + written + index list), 185k-row prefix"


def relocation_workload(seed: int = 77) -> dict:
    """The relocation benchmark's inputs (same recipe as its GPU parity test)."""
    rng = np.random.default_rng(seed)
    pool = rng.integers(0, 1 << 16, size=(RELOC_SLOTS, 576), dtype=np.uint16)  # a bytewise copy: any bits
    idx = rng.choice(RELOC_SLOTS // 2, size=RELOC_PREFIX + RELOC_T, replace=False).astype(np.int32)
    return dict(pool=pool, kv_indices=idx, prefix_lens=np.array([RELOC_PREFIX], dtype=np.int32),
                dst_start=np.array([RELOC_SLOTS // 2 + 12345], dtype=np.int32))


def relocation_bytes() -> int:
    """Algorithmic bytes of one relocation: each row read and written once, and the prefix
    part of the index list read and rewritten."""
    return RELOC_PREFIX * (2 * KV_ROW_BYTES + 2 * INDEX_BYTES)


def bench_relocate(args) -> int:
    import torch

    import mla_tree_verify_mlaverify_amd as mv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = relocation_workload()
    pool = torch.from_numpy(w["pool"].view(np.int16)).view(torch.bfloat16).to(dev)
    idx0 = torch.from_numpy(w["kv_indices"]).to(dev)
    idx = idx0.clone()
    plens = torch.from_numpy(w["prefix_lens"]).to(dev)
    dst = torch.from_numpy(w["dst_start"]).to(dev)
    v = mv.Verifier(num_heads=8, max_batch=1, max_tree_nodes=RELOC_T, max_prefix_len=RELOC_PREFIX,
                    pool_slots=RELOC_SLOTS, device=dev)
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        idx.copy_(idx0)
        if not args.warm:
            flush.add_(1.0)
        v.relocate(pool, idx, plens, dst, RELOC_T, stream=stream)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    wall0 = time.perf_counter()
    for k in range(args.steps):
        idx.copy_(idx0)
        if not args.warm:
            flush.add_(1.0)
        starts[k].record(stream)
        v.relocate(pool, idx, plens, dst, RELOC_T, stream=stream)
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    assert v.read_device_errors() == 0
    d0 = int(w["dst_start"][0])
    assert torch.equal(idx[:RELOC_PREFIX].cpu(), torch.arange(d0, d0 + RELOC_PREFIX, dtype=torch.int32))
    call_ms = [s_.elapsed_time(e) for s_, e in zip(starts, ends)]
    med_ms = statistics.median(call_ms)
    nbytes = relocation_bytes()
    gbs = nbytes / (med_ms * 1e-3) / 1e9
    line = {
        "metric": RELOC_METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": f"relocate_p{RELOC_PREFIX}_pool{RELOC_SLOTS}", "prefix": RELOC_PREFIX,
                   "tree_nodes": RELOC_T, "pool_slots": RELOC_SLOTS,
                   "cache": "warm" if args.warm else "flushed 1 GiB before each call"},
        "us_per_call": {"median": round(med_ms * 1e3, 2), "p10": round(float(np.percentile(call_ms, 10)) * 1e3, 2),
                        "p90": round(float(np.percentile(call_ms, 90)) * 1e3, 2)},
        "wall_s_timed_loop": round(wall, 4),
        # the four launches of one call (prepare, mark, check, copy) timed together: the copy
        # dominates, so the call is held to the copy's HBM roofline
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "k_reloc_* (one call)",
                     "kernel_avg_us": round(1e3 * sum(call_ms) / len(call_ms), 2)},
    }
    if not args.no_cpu:
        from oracle import relocate_oracle as rel

        t0 = time.perf_counter()
        _, _, err = rel.relocate(w["pool"], w["kv_indices"], w["prefix_lens"], RELOC_T, w["dst_start"],
                                 RELOC_PREFIX)
        secs = time.perf_counter() - t0
        assert err == 0
        line["cpu_baseline"] = {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                                "sample": f"one whole relocation of the same workload ({secs:.2f} s)",
                                "cpu_model": lscpu_model()}
    print(json.dumps(line), flush=True)
    return 0


ACCEPT_B, ACCEPT_T, ACCEPT_V = 1, 64, 131072
ACCEPT_METRIC = "tree-acceptance GB/s (fp32 logits read), 64-node tree, 131,072-token vocabulary"


def bench_accept(args) -> int:
    import torch

    import mla_tree_verify_mlaverify_amd as mv
    from workloads import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.accept_config(0, batch=ACCEPT_B, tree_nodes=ACCEPT_T, vocab=ACCEPT_V)
    logits = torch.from_numpy(cfg["logits"]).to(dev)
    tokens = torch.from_numpy(cfg["draft_tokens"]).to(dev)
    parents = torch.from_numpy(cfg["tree_parent"]).to(dev)
    v = mv.Verifier(num_heads=1, max_batch=ACCEPT_B, max_tree_nodes=ACCEPT_T, max_prefix_len=1, pool_slots=1,
                    device=dev)
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        if not args.warm:
            flush.add_(1.0)
        v.accept(logits, tokens, parents, stream=stream)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    wall0 = time.perf_counter()
    for k in range(args.steps):
        if not args.warm:
            flush.add_(1.0)
        starts[k].record(stream)
        lens, _, _ = v.accept(logits, tokens, parents, stream=stream)
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    assert v.read_device_errors() == 0
    call_ms = [s_.elapsed_time(e) for s_, e in zip(starts, ends)]
    med_ms = statistics.median(call_ms)
    nbytes = ACCEPT_B * (ACCEPT_T + 1) * ACCEPT_V * 4
    gbs = nbytes / (med_ms * 1e-3) / 1e9
    line = {
        "metric": ACCEPT_METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(med_ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": f"accept_b{ACCEPT_B}_t{ACCEPT_T}_v{ACCEPT_V}", "batch": ACCEPT_B,
                   "tree_nodes": ACCEPT_T, "vocab": ACCEPT_V, "accepted": int(lens[0]),
                   "cache": "warm" if args.warm else "flushed 1 GiB before each call"},
        "us_per_call": {"median": round(med_ms * 1e3, 2), "p10": round(float(np.percentile(call_ms, 10)) * 1e3, 2),
                        "p90": round(float(np.percentile(call_ms, 90)) * 1e3, 2)},
        "wall_s_timed_loop": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "k_accept_* (one call)",
                     "kernel_avg_us": round(1e3 * sum(call_ms) / len(call_ms), 2)},
    }
    if not args.no_cpu:
        from oracle import accept_oracle as acc

        t0 = time.perf_counter()
        acc.accept(cfg["logits"], cfg["draft_tokens"], cfg["tree_parent"])
        secs = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                                "sample": f"one whole call on the same inputs ({secs:.3f} s); the oracle takes the argmax "
                                          "only of the rows its walk visits, the GPU of every row",
                                "cpu_model": lscpu_model()}
    print(json.dumps(line), flush=True)
    return 0


RAGGED_SEED = 5
RAGGED_METRIC = ("ragged verify µs/call (a tree size per request) against the same batch padded to its "
                 "largest tree, 8 requests, 1k-131k prefixes, 16 heads")


def ragged_workload(seed: int = RAGGED_SEED):
    """The batch-of-8 workload (1k-131k prefixes, 32-node trees, 16 heads) with a tree size
    drawn per request, uniform in 4..32 (the first request keeps all 32, so the padded call
    has the same largest tree).  A request of T_b nodes keeps the first T_b nodes of its tree
    (parents precede children, so they form a tree), their query rows and the first T_b tree
    slots of its index segment.  Returns (the padded workload, the packed ragged arrays)."""
    from workloads import synth

    cfg = synth.make_config(4)
    B, T, H = cfg["batch"], cfg["tree_nodes"], cfg["heads"]
    tl = np.random.default_rng(seed).integers(4, T + 1, size=B).astype(np.int32)
    tl[0] = T
    plens = cfg["prefix_lens"].astype(np.int64)
    offs = synth.request_offsets(plens, T)
    q = cfg["q"].reshape(B, T, H, -1)
    rag = dict(
        q=np.concatenate([q[b, : tl[b]] for b in range(B)]),
        kv_indices=np.concatenate([cfg["kv_indices"][offs[b]: offs[b] + plens[b] + tl[b]] for b in range(B)]
                                  ).astype(np.int32),
        prefix_lens=cfg["prefix_lens"].astype(np.int32),
        tree_lens=tl,
        tree_parent=np.concatenate([cfg["tree_parent"][b, : tl[b]] for b in range(B)]).astype(np.int32))
    return cfg, rag


def ragged_counts(cfg: dict, rag: dict) -> dict:
    """Algorithmic bytes and flops of the ragged call: each request's prefix and its T_b tree
    keys read once; 2 H (576 + 512) flops per visible (row, key) pair."""
    from workloads import synth

    h = cfg["heads"]
    plens = rag["prefix_lens"].astype(np.int64)
    tl = rag["tree_lens"].astype(np.int64)
    keys = int(plens.sum() + tl.sum())
    rows = int(tl.sum())
    visible, o = 0, 0
    for b in range(len(tl)):
        depth = synth.tree_depths(rag["tree_parent"][o: o + tl[b]])
        visible += int(tl[b] * plens[b]) + int((depth + 1).sum())
        o += int(tl[b])
    total = keys * (KV_ROW_BYTES + INDEX_BYTES) + rows * h * (576 * 2 + 512 * 2 + 4)
    return dict(keys=keys, kv_bytes=keys * KV_ROW_BYTES, total_bytes=total, flops=2 * h * visible * (576 + 512))


def time_ragged(steps: int, warmup: int, warm: bool, flush) -> dict:
    """Times the ragged call (mlaverify_run_ragged) and the padded call (mlaverify_run on the
    same batch with every request at the largest tree) with the verify protocol: clock settle,
    warmup, caches flushed before each call, one event pair per call, then the library's
    per-kernel events.  Returns both summaries, the speedup and the workload."""
    import torch

    import mla_tree_verify_mlaverify_amd as mv

    dev = flush.device
    cfg, rag = ragged_workload()
    B, T, H = cfg["batch"], cfg["tree_nodes"], cfg["heads"]

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    pool = bf16(cfg["pool"])
    plens = i32(cfg["prefix_lens"])
    v = mv.Verifier(num_heads=H, max_batch=B, max_tree_nodes=T, max_prefix_len=int(cfg["prefix_lens"].max()),
                    pool_slots=cfg["slots"], sm_scale=cfg["sm_scale"], device=dev)
    stream = torch.cuda.current_stream()
    pq, pidx, ppar = bf16(cfg["q"]), i32(cfg["kv_indices"]), i32(cfg["tree_parent"])
    pout = torch.empty((B * T, H, 512), dtype=torch.bfloat16, device=dev)
    plse = torch.empty((B * T, H), dtype=torch.float32, device=dev)
    rows = int(rag["tree_lens"].sum())
    rq, ridx, rtl, rpar = bf16(rag["q"]), i32(rag["kv_indices"]), i32(rag["tree_lens"]), i32(rag["tree_parent"])
    rout = torch.empty((rows, H, 512), dtype=torch.bfloat16, device=dev)
    rlse = torch.empty((rows, H), dtype=torch.float32, device=dev)

    def padded():
        v.run(pq, pool, pidx, plens, ppar, out=pout, lse=plse, stream=stream)

    def ragged():
        v.run_ragged(rq, pool, ridx, plens, rtl, rpar, T, out=rout, lse=rlse, stream=stream)

    res = {}
    for name, step in (("ragged", ragged), ("padded", padded)):
        settle(step, flush, warm)
        for _ in range(warmup):
            if not warm:
                flush.add_(1.0)
            step()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        for k in range(steps):
            if not warm:
                flush.add_(1.0)
            starts[k].record(stream)
            step()
            ends[k].record(stream)
        torch.cuda.synchronize()
        call_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
        v.profile_begin(steps)
        for _ in range(steps):
            if not warm:
                flush.add_(1.0)
            step()
        torch.cuda.synchronize()
        kms = v.profile_end()
        res[name] = dict(call_ms=call_ms, med=statistics.median(call_ms),
                         part=sum(k[0] for k in kms) / len(kms), merge=sum(k[1] for k in kms) / len(kms))
    assert v.read_device_errors() == 0
    # the ragged rows equal the padded call's rows of the nodes they keep (bit for bit: the
    # plan differs, so only up to the partials' rounding)
    o = 0
    worst = 0.0
    for b in range(B):
        t_b = int(rag["tree_lens"][b])
        d = (rout[o: o + t_b].float() - pout[b * T: b * T + t_b].float()).abs().max().item()
        worst = max(worst, d)
        o += t_b
    rc = ragged_counts(cfg, rag)
    pc = algorithmic_counts(cfg)

    def summary(r, counts):
        t_hbm = counts["total_bytes"] / (HBM_PEAK_GBS * 1e9)
        t_mfma = counts["flops"] / (BF16_MFMA_PEAK_TFLOPS * 1e12)
        part_s = r["part"] * 1e-3
        if t_mfma >= t_hbm:
            ach = counts["flops"] / part_s / 1e12
            roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / BF16_MFMA_PEAK_TFLOPS, 4)}
        else:
            ach = counts["total_bytes"] / part_s / 1e9
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4)}
        roof.update(traffic=None, kernel="k_partial", kernel_avg_us=round(r["part"] * 1e3, 2))
        return {"us_per_call": {"median": round(r["med"] * 1e3, 2),
                                "p10": round(float(np.percentile(r["call_ms"], 10)) * 1e3, 2),
                                "p90": round(float(np.percentile(r["call_ms"], 90)) * 1e3, 2)},
                "kernels_us": {"partial": round(r["part"] * 1e3, 2), "merge": round(r["merge"] * 1e3, 2)},
                "kv_gbs": round(counts["kv_bytes"] / (r["med"] * 1e-3) / 1e9, 2),
                "gflop": round(counts["flops"] / 1e9, 2), "roofline": roof}

    rs, ps = summary(res["ragged"], rc), summary(res["padded"], pc)
    name = f"ragged_b{B}_ploguniform_t4to{T}_h{H}"
    if not warm:  # HBM bytes per launch of the ragged call from its committed counters
        rs["roofline"]["traffic"] = stored_traffic(name)
        rs["profile"] = f"profiles/k_partial_{name}.md" if rs["roofline"]["traffic"] else None
    del v
    torch.cuda.empty_cache()
    return {"config": {"workload": name, "batch": B, "heads": H,
                       "tree_lens": [int(x) for x in rag["tree_lens"]],
                       "prefix_lens": [int(x) for x in cfg["prefix_lens"]],
                       "cache": "warm" if warm else "flushed 1 GiB before each call"},
            "ragged": rs, "padded": ps,
            "speedup_vs_padded": round(res["padded"]["med"] / res["ragged"]["med"], 3),
            "rows": {"ragged": rows * H, "padded": B * T * H},
            "max_abs_diff_vs_padded_rows": worst, "steps": steps,
            "ms_per_step": round(res["ragged"]["med"], 5)}


def bench_ragged(args) -> int:
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    r = time_ragged(args.steps, args.warmup, args.warm, flush)
    line = {
        "metric": RAGGED_METRIC, "value": r["ragged"]["us_per_call"]["median"], "unit": "us/call", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": r["config"], "ragged": r["ragged"], "padded": r["padded"],
        "speedup_vs_padded": r["speedup_vs_padded"], "rows": r["rows"],
        "max_abs_diff_vs_padded_rows": r["max_abs_diff_vs_padded_rows"],
        "roofline": r["ragged"]["roofline"],
    }
    print(json.dumps(line), flush=True)
    return 0


GATHER_METRIC = "scattered KV-row gather GB/s (185,000 rows of 1,152 B from a 262,144-slot pool, caches flushed)"
GATHER_GRIDS = (256, 512, 1024, 2048)


def gather_probe(cfg: dict, flush, grids=GATHER_GRIDS, reps: int = 10) -> dict:
    """Rate of the probe kernels (mlaverify_probe_gather) reading the workload's prefix rows through
    each 16-byte load path, per grid size: {"register": {grid: GB/s}, "lds": {...}} counting the
    rows' 1,152 bytes (the index list adds 4 bytes per row)."""
    import torch

    import mla_tree_verify_mlaverify_amd as mv

    dev = flush.device
    p = int(cfg["prefix_lens"][0])
    pool = torch.from_numpy(np.ascontiguousarray(cfg["pool"]).view(np.int16)).view(torch.bfloat16).to(dev)
    idx = torch.from_numpy(np.ascontiguousarray(cfg["kv_indices"][:p], dtype=np.int32)).to(dev)
    out = {}
    for name, lds in (("register", False), ("lds", True)):
        out[name] = {}
        for g in grids:
            sink = torch.empty(g * 256, dtype=torch.int32, device=dev)
            for _ in range(2):
                flush.add_(1.0)
                mv.probe_gather(pool, idx, lds, g, sink)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for a, b in ev:
                flush.add_(1.0)
                a.record()
                mv.probe_gather(pool, idx, lds, g, sink)
                b.record()
            torch.cuda.synchronize()
            ms = statistics.median(a.elapsed_time(b) for a, b in ev)
            out[name][str(g)] = round(p * KV_ROW_BYTES / (ms * 1e-3) / 1e9, 1)
    return out


def bench_gather(args) -> int:
    import torch

    from workloads import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.make_config(3)
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    copy_gbs = stream_bandwidth(flush)
    t0 = time.perf_counter()
    rates = gather_probe(cfg, flush, reps=args.steps)
    wall = time.perf_counter() - t0
    best = max(rates["register"].values())
    p = int(cfg["prefix_lens"][0])
    line = {
        "metric": GATHER_METRIC, "value": best, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": 2,
        "ms_per_step": round(p * KV_ROW_BYTES / (best * 1e9) * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": "gather_p185000_pool262144", "rows": p, "row_bytes": KV_ROW_BYTES,
                   "pool_slots": cfg["slots"], "indices": "the 185k workload's scattered prefix slots",
                   "threads_per_row": 8, "loads_in_flight_per_thread": 36},
        "rates_gbs": rates, "hbm_stream_gbs": round(copy_gbs, 1),
        "pct_hbm_measured": round(100 * best / copy_gbs, 2),
        "wall_s_timed_loop": round(wall, 3),
        "roofline": {"bound": "hbm", "achieved": best, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(best / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "k_probe_gather<register>"},
    }
    if not args.no_cpu:
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 3.0:
            cfg["pool"][cfg["kv_indices"][:p]].sum(dtype=np.uint64)
            reps += 1
        secs = (time.perf_counter() - t0) / reps
        line["cpu_baseline"] = {"value": round(p * KV_ROW_BYTES / secs / 1e9, 3), "unit": "GB/s", "cores": 1,
                                "kind": "numpy gather", "sample": f"pool[indices] of the same rows, {reps} times",
                                "cpu_model": lscpu_model()}
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload index (workloads.synth.CONFIGS)")
    ap.add_argument("--variant", default=None,
                    help="workload variant, e.g. contiguous or sorted, or unit_end_needles (a dominant key at the "
                         "last prefix key of every split unit)")
    ap.add_argument("--warm", action="store_true", help="do not flush caches between calls")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the call captured in a HIP graph (the flush stays outside it)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--split", type=int, default=0, help="fixed split length (0 = automatic)")
    ap.add_argument("--op", choices=("verify", "relocate", "accept", "gather", "ragged"), default="verify")
    ap.add_argument("--page", type=int, default=0, help="prefix page size (block table of page ids); 0 = per token")
    ap.add_argument("--no-per-config", action="store_true",
                    help="time only the chosen workload (by default the 185k run also times every other one)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2
    if args.op == "relocate":
        return bench_relocate(args)
    if args.op == "accept":
        return bench_accept(args)
    if args.op == "gather":
        return bench_gather(args)
    if args.op == "ragged":
        return bench_ragged(args)

    import torch

    import mla_tree_verify_mlaverify_amd as mv
    from workloads import synth

    if not os.path.exists(mv.LIB_PATH):
        raise SystemExit(f"{mv.LIB_PATH} not built: run `python -m mla_tree_verify_mlaverify_amd.build`")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB, read and written before each call
    copy_gbs = stream_bandwidth(flush)

    cfg, workload = verify_workload(args.config, args.variant, args.page)
    res = time_verify(cfg, args, flush, args.steps, args.warmup, graph=args.graph, split=args.split, page=args.page)
    counts = algorithmic_counts(cfg)
    summ = verify_summary(cfg, counts, res, copy_gbs)
    med_ms = res["call_ms_median"]
    roof = summ["roofline"]
    roof["traffic"] = (stored_traffic(synth.CONFIGS[args.config]["name"])
                       if not (args.variant or args.split or args.warm or args.page > 1) else None)
    line = {
        "metric": METRIC,
        "value": summ["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload,
                   "batch": cfg["batch"], "tree_nodes": cfg["tree_nodes"], "heads": cfg["heads"],
                   "prefix_lens": [int(x) for x in cfg["prefix_lens"]], "pool_slots": cfg["slots"],
                   "split": args.split or "auto", "cache": "warm" if args.warm else "flushed 1 GiB before each call",
                   "call": "HIP graph replay" if args.graph else "eager"},
        "wall_s_timed_loop": res["wall_s"],
        "hbm_stream_gbs": round(copy_gbs, 1),
    }
    line.update({k: summ[k] for k in ("us_per_call", "kernels_us", "pct_hbm_peak", "pct_hbm_measured", "tflops",
                                      "pct_mfma_peak", "roofline_frac_call", "sclk_mhz", "plan")})
    line["roofline"] = roof
    if not (args.variant or args.split or args.warm or args.page > 1):
        line.update(profile_fields(synth.CONFIGS[args.config]["name"]))
    del res
    if not args.no_per_config and args.config == 3 and not (args.variant or args.page > 1 or args.split):
        # the other seeded workloads, timed in the same run with the same protocol (fewer calls)
        per = {}
        steps = max(10, args.steps // 2)
        for i, var in PER_CONFIG:
            c, name = verify_workload(i, var, 0)
            r = time_verify(c, args, flush, steps, min(args.warmup, 3), graph=False, split=0, page=0)
            per[name] = verify_summary(c, algorithmic_counts(c), r, copy_gbs)
            per[name]["steps"] = steps
            if var is None:
                per[name].update(profile_fields(name))
                per[name]["roofline"]["traffic"] = stored_traffic(name)
            del r, c
            torch.cuda.empty_cache()
        line["per_config"] = per
        # the ragged batch (a tree size per request) against the same batch padded
        line["ragged"] = time_ragged(steps, min(args.warmup, 3), args.warm, flush)
        # the scattered-read ceiling of the two load paths on the headline's own rows
        line["gather_probe_gbs"] = gather_probe(cfg, flush, grids=(512,))
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(cfg, counts, args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


# The seeded workloads other than the 185k headline, each timed once per default run: the
# 4k and 65k prefixes (the 65k one also with its indices sorted, and as one contiguous run),
# the batch of 8, and the two HBM-bound small-tree shapes (each also as one contiguous run,
# where the fast path's savings would show first).
PER_CONFIG = [(1, None), (2, None), (2, "sorted"), (2, "contiguous"), (4, None), (5, None), (5, "contiguous"),
              (6, None), (6, "contiguous")]


def verify_workload(i: int, variant, page: int):
    from workloads import synth

    if variant == "unit_end_needles":
        # a dominant key at the last prefix key of every split unit (the automatic split of
        # this workload, read back from one call): the worst place for a raised reference
        cfg = synth.make_config(i)
        cfg = synth.plant_unit_end_needles(cfg, automatic_split(cfg))
    else:
        cfg = synth.make_config(i, variant=variant)
    name = synth.CONFIGS[i]["name"] + (f"+{variant}" if variant else "")
    if page > 1:  # the same shapes with paged prefixes (pages drawn at random, tree slots apart)
        cfg = synth.paged_config(i, batch=cfg["batch"], prefix=[int(p) for p in cfg["prefix_lens"]],
                                 tree_nodes=cfg["tree_nodes"], heads=cfg["heads"], slots=cfg["slots"], page=page)
        name += f"+paged{page}"
    return cfg, name


def automatic_split(cfg: dict) -> int:
    """The split length the library's automatic plan picks for this workload (one call)."""
    import torch

    import mla_tree_verify_mlaverify_amd as mv

    dev = torch.device("cuda:0")

    def t(a, dt=None):
        x = torch.from_numpy(np.ascontiguousarray(a if dt is None else a.astype(dt)))
        return (x.view(torch.int16).view(torch.bfloat16) if dt is None else x).to(dev)

    v = mv.Verifier(num_heads=cfg["heads"], max_batch=cfg["batch"], max_tree_nodes=cfg["tree_nodes"],
                    max_prefix_len=int(cfg["prefix_lens"].max()), pool_slots=cfg["slots"], sm_scale=cfg["sm_scale"],
                    device=dev)
    v.run(t(cfg["q"].view(np.int16)), t(cfg["pool"].view(np.int16)), t(cfg["kv_indices"], np.int32),
          t(cfg["prefix_lens"], np.int32), t(cfg["tree_parent"], np.int32))
    return v.read_plan()["split_len"]


def stream_bandwidth(flush) -> float:
    """Measured HBM rate of a plain streaming kernel: the 1 GiB read-modify-write used as the cache
    flush (2 GiB of traffic per launch), median of 10 launches, GB/s."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(12)]
    for a, b in ev:
        a.record()
        flush.add_(1.0)
        b.record()
    torch.cuda.synchronize()
    ms = statistics.median(a.elapsed_time(b) for a, b in ev[2:])
    return 2 * flush.numel() * 4 / (ms * 1e-3) / 1e9


SETTLE_S = 0.3


def settle(step, flush, warm: bool) -> None:
    """Clock settle before the warmup steps: back-to-back calls (with the flush unless warm) for
    SETTLE_S seconds.  The GPU's clocks take tens of milliseconds of load to ramp up, so with
    only a few warmup calls the first timed calls ran several percent slower (measured: 185k
    workload, 5 warmup calls, call median 206.6 µs and p90 224 µs; 40 calls, 195.7 and 196.5)."""
    import torch

    t0 = time.perf_counter()
    n = 0
    while n < 2000 and (n % 8 or time.perf_counter() - t0 < SETTLE_S):
        if not warm:
            flush.add_(1.0)
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_verify(cfg: dict, args, flush, steps: int, warmup: int, *, graph: bool, split: int, page: int) -> dict:
    """Upload one workload, then time `steps` whole calls (one HIP event pair around each, caches
    flushed before each unless --warm) and `steps` more with the library's events around each
    kernel.  Returns per-call milliseconds, per-kernel milliseconds and the plan."""
    import torch

    import mla_tree_verify_mlaverify_amd as mv

    dev = flush.device

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    q, pool = bf16(cfg["q"]), bf16(cfg["pool"])
    kv_idx, plens, par = i32(cfg["kv_indices"]), i32(cfg["prefix_lens"]), i32(cfg["tree_parent"])
    v = mv.Verifier(num_heads=cfg["heads"], max_batch=cfg["batch"], max_tree_nodes=cfg["tree_nodes"],
                    max_prefix_len=int(cfg["prefix_lens"].max()), pool_slots=cfg["slots"],
                    sm_scale=cfg["sm_scale"], split_tokens=split, page_size=page, device=dev)
    b, t, h = cfg["batch"], cfg["tree_nodes"], cfg["heads"]
    out = torch.empty((b * t, h, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((b * t, h), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        v.run(q, pool, kv_idx, plens, par, out=out, lse=lse, stream=stream)

    settle(step, flush, args.warm)
    for _ in range(warmup):
        if not args.warm:
            flush.add_(1.0)
        step()
    torch.cuda.synchronize()
    call = step
    if graph:  # the same call, captured once on a side stream and replayed on this one
        gs = torch.cuda.Stream(device=dev)
        gs.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            v.run(q, pool, kv_idx, plens, par, out=out, lse=lse, stream=gs)
        torch.cuda.synchronize()
        call = g.replay
        for _ in range(warmup):
            if not args.warm:
                flush.add_(1.0)
            call()
        torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    v.read_plan(stream=stream)  # (sets the rescale count back to 0 for the timed calls)
    # Whole calls, timed on their own: the library's per-kernel events (below) would add
    # their own markers between the two launches.
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(steps):
        if not args.warm:
            flush.add_(1.0)
        starts[k].record(stream)
        call()
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    call_ms = [s_.elapsed_time(e) for s_, e in zip(starts, ends)]
    # The same calls again with the library's HIP events around each of its kernels.
    v.profile_begin(steps)
    for _ in range(steps):
        if not args.warm:
            flush.add_(1.0)
        step()
    torch.cuda.synchronize()
    kernel_ms = v.profile_end()
    errs = v.read_device_errors()
    assert errs == 0, errs
    plan = v.read_plan()
    plan["rescales_per_call"] = plan["rescales"] / (2 * steps)
    return dict(call_ms=call_ms, call_ms_median=statistics.median(call_ms), kernel_ms=kernel_ms, plan=plan,
                wall_s=round(wall, 4))


def verify_summary(cfg: dict, counts: dict, res: dict, copy_gbs: float) -> dict:
    """The metric's figures for one timed workload: µs per call, KV GB/s and %HBM (of the nominal
    peak and of the measured stream rate), %MFMA, and the partial kernel's roofline."""
    call_ms = res["call_ms"]
    med_ms = res["call_ms_median"]
    part_ms = [k[0] for k in res["kernel_ms"]]
    merge_ms = [k[1] for k in res["kernel_ms"]]
    part_avg = sum(part_ms) / len(part_ms)
    kv_gbs = counts["kv_bytes"] / (med_ms * 1e-3) / 1e9
    tflops = counts["flops"] / (med_ms * 1e-3) / 1e12
    t_hbm = counts["total_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = counts["flops"] / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    if t_mfma >= t_hbm:
        ach = counts["flops"] / (part_avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None}
    else:
        ach = counts["total_bytes"] / (part_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}
    roof["kernel"] = "k_partial"
    roof["kernel_avg_us"] = round(part_avg * 1e3, 2)
    plan = res["plan"]
    s = plan["split_len"]
    prefix_units = sum(min(r["units"], -(-r["prefix_len"] // s)) for r in plan["requests"])
    return {
        "us_per_call": {"median": round(med_ms * 1e3, 2), "p10": round(float(np.percentile(call_ms, 10)) * 1e3, 2),
                        "p90": round(float(np.percentile(call_ms, 90)) * 1e3, 2)},
        "kernels_us": {"partial": round(part_avg * 1e3, 2), "merge": round(1e3 * sum(merge_ms) / len(merge_ms), 2),
                       "call_minus_partial": round(med_ms * 1e3 - part_avg * 1e3, 2)},
        "kv_gbs": round(kv_gbs, 2),
        "pct_hbm_peak": round(100 * kv_gbs / HBM_PEAK_GBS, 2),
        "pct_hbm_measured": round(100 * kv_gbs / copy_gbs, 2),
        "tflops": round(tflops, 2),
        "pct_mfma_peak": round(100 * tflops / BF16_MFMA_PEAK_TFLOPS, 2),
        "roofline_frac_call": round(max(t_hbm, t_mfma) / (med_ms * 1e-3), 4),
        "sclk_mhz": plan.get("sclk_mhz"),
        "roofline": roof,
        "plan": {"split_len": s, "total_units": plan["total_units"], "n_mtiles": plan["n_mtiles"],
                 "fast_units": plan["fast_units"], "prefix_units": prefix_units,
                 "fast_hit_rate": round(plan["fast_units"] / prefix_units, 4) if prefix_units else None,
                 "rescales_per_call": plan["rescales_per_call"]},
    }


if __name__ == "__main__":
    sys.exit(main())
