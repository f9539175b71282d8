"""Benchmark of DDTree MLA tree-verify attention on one MI355X.

One step = one full verify pass (plan + split-KV partials + LSE merge) over the
workload, with its inputs resident in HBM and the caches flushed before each call
(a 1 GiB read-modify-write), since a long-context KV does not stay cached between
decode steps.  Prints one JSON line; see the design doc for the fields.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--config 3] [--warm] [--no-cpu]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

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
    total_bytes = kv_bytes + keys * INDEX_BYTES + q_bytes + out_bytes
    visible = 0  # sum over (request, node) of |prefix| + |ancestors incl. self|
    for bb in range(b):
        depth = synth.tree_depths(cfg["tree_parent"][bb])
        visible += t * int(plens[bb]) + int((depth + 1).sum())
    flops = 2 * h * visible * (576 + 512)
    return dict(keys=keys, kv_bytes=kv_bytes, total_bytes=total_bytes, flops=flops,
                prefix_flops=2 * h * t * int(plens.sum()) * (576 + 512))


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

    try:
        from threadpoolctl import threadpool_info

        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=os.cpu_count())
    except Exception:
        threads = os.cpu_count()
    t_nodes = cfg["tree_nodes"]
    # time one node of request 0 first, then size the sample to the budget
    t0 = time.perf_counter()
    orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"], cfg["tree_parent"],
                         cfg["sm_scale"], nodes=[(0, 0)])
    one = time.perf_counter() - t0
    n_nodes = int(max(1, min(t_nodes * cfg["batch"], budget_s / max(one, 1e-3))))
    nodes = [(bb, i) for bb in range(cfg["batch"]) for i in range(t_nodes)][:n_nodes]
    t0 = time.perf_counter()
    orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"], cfg["tree_parent"],
                         cfg["sm_scale"], nodes=nodes)
    secs = time.perf_counter() - t0
    frac = len(nodes) / (t_nodes * cfg["batch"])
    est_call_s = secs / frac
    return {"value": round(counts["kv_bytes"] / est_call_s / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(nodes)} of {t_nodes * cfg['batch']} tree nodes (all heads) of the same workload, "
                      f"{secs:.1f} s; per-call time scaled by the node fraction ({est_call_s:.2f} s/call)",
            "cpu_model": lscpu_model()}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, help="workload index (workloads.synth.CONFIGS)")
    ap.add_argument("--variant", default=None, help="workload variant, e.g. contiguous or sorted")
    ap.add_argument("--warm", action="store_true", help="do not flush caches between calls")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--split", type=int, default=0, help="fixed split length (0 = automatic)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import mla_tree_verify_mlaverify_amd as mv
    from workloads import synth

    if not os.path.exists(mv.LIB_PATH):
        raise SystemExit(f"{mv.LIB_PATH} not built: run `python -m mla_tree_verify_mlaverify_amd.build`")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.make_config(args.config, variant=args.variant)
    counts = algorithmic_counts(cfg)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    q, pool = bf16(cfg["q"]), bf16(cfg["pool"])
    kv_idx, plens, par = i32(cfg["kv_indices"]), i32(cfg["prefix_lens"]), i32(cfg["tree_parent"])
    v = mv.Verifier(num_heads=cfg["heads"], max_batch=cfg["batch"], max_tree_nodes=cfg["tree_nodes"],
                    max_prefix_len=int(cfg["prefix_lens"].max()), pool_slots=cfg["slots"],
                    sm_scale=cfg["sm_scale"], split_tokens=args.split, device=dev)
    b, t, h = cfg["batch"], cfg["tree_nodes"], cfg["heads"]
    out = torch.empty((b * t, h, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((b * t, h), dtype=torch.float32, device=dev)
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    stream = torch.cuda.current_stream()

    def step():
        v.run(q, pool, kv_idx, plens, par, out=out, lse=lse, stream=stream)

    for _ in range(args.warmup):
        if not args.warm:
            flush.add_(1.0)
        step()
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    v.profile_begin(args.steps)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(args.steps):
        if not args.warm:
            flush.add_(1.0)
        starts[k].record(stream)
        step()
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    kernel_ms = v.profile_end()
    call_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    errs = v.read_device_errors()
    assert errs == 0, errs

    med_ms = statistics.median(call_ms)
    p10, p90 = np.percentile(call_ms, 10), np.percentile(call_ms, 90)
    part_ms = [k[0] for k in kernel_ms]
    part_avg = sum(part_ms) / len(part_ms)
    kv_gbs = counts["kv_bytes"] / (med_ms * 1e-3) / 1e9
    tflops = counts["flops"] / (med_ms * 1e-3) / 1e12
    part_tflops = counts["flops"] / (part_avg * 1e-3) / 1e12
    t_hbm = counts["total_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = counts["flops"] / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(part_tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(part_tflops / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None}
    else:
        part_gbs = counts["total_bytes"] / (part_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(part_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(part_gbs / HBM_PEAK_GBS, 4), "traffic": None}
    roof["kernel"] = "k_partial"
    roof["kernel_avg_us"] = round(part_avg * 1e3, 2)

    line = {
        "metric": "verify-attn KV GB/s (64-node tree, 185k prefix)" if args.config == 3 else
                  f"verify-attn KV GB/s ({synth.CONFIGS[args.config]['name']})",
        "value": round(kv_gbs, 2),
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
        "config": {"workload": synth.CONFIGS[args.config]["name"] + (f"+{args.variant}" if args.variant else ""),
                   "batch": b, "tree_nodes": t, "heads": h,
                   "prefix_lens": [int(x) for x in cfg["prefix_lens"]], "pool_slots": cfg["slots"],
                   "split": args.split or "auto", "cache": "warm" if args.warm else "flushed 1 GiB before each call"},
        "us_per_call": {"median": round(med_ms * 1e3, 2), "p10": round(float(p10) * 1e3, 2),
                        "p90": round(float(p90) * 1e3, 2)},
        "pct_hbm_peak": round(100 * kv_gbs / HBM_PEAK_GBS, 2),
        "tflops": round(tflops, 2),
        "pct_mfma_peak": round(100 * tflops / BF16_MFMA_PEAK_TFLOPS, 2),
        "roofline_frac_call": round(max(t_hbm, t_mfma) / (med_ms * 1e-3), 4),
        "kernels_us": {"partial": round(part_avg * 1e3, 2),
                       "merge": round(1e3 * sum(k[1] for k in kernel_ms) / len(kernel_ms), 2)},
        "wall_s_timed_loop": round(wall, 4),
        "roofline": roof,
        "plan": {k: v.read_plan()[k] for k in ("split_len", "total_units", "n_mtiles")},
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(cfg, counts, args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
