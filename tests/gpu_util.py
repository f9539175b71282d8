"""Shared helpers of the GPU tests: upload a synthetic workload, run the HIP library
through its C ABI binding, compare against the CPU fp64 oracle."""

from __future__ import annotations

import numpy as np
import torch

import mla_tree_verify_mlaverify_amd as mv
from oracle import mla_tree_oracle as orc

DEV = torch.device("cuda:0")

# Contract tolerance on the bf16 output and the fp32 lse.
OUT_ATOL = 1e-2
OUT_RTOL = 1e-2
LSE_ATOL = 1e-3
# Stricter bar, from the arithmetic: P is rounded to bf16 before the PV product (relative
# error <= 2^-9 per weight) and the output is rounded to bf16 (<= 2^-9), so the error of a
# row, measured in its own L2 norm, stays below 2 * 2^-9 ~ 3.9e-3 plus fp32 accumulation
# noise; 1e-2 leaves margin.  The lse is formed in fp32 (relative 1e-6 of |lse| per step).
ROW_REL_L2 = 1e-2
LSE_ABS_STRICT = 2e-4


def bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def upload(cfg: dict) -> dict:
    return dict(q=bf16(cfg["q"]), pool=bf16(cfg["pool"]), kv_indices=i32(cfg["kv_indices"]),
                prefix_lens=i32(cfg["prefix_lens"]), tree_parent=i32(cfg["tree_parent"]))


def verifier_for(cfg: dict, *, max_batch=None, max_prefix=None, **kw) -> mv.Verifier:
    return mv.Verifier(num_heads=cfg["heads"], max_batch=max_batch or cfg["batch"],
                       max_tree_nodes=cfg["tree_nodes"],
                       max_prefix_len=max_prefix if max_prefix is not None else max(1, int(cfg["prefix_lens"].max())),
                       pool_slots=cfg["slots"], kv_row_stride=cfg["row_stride"], sm_scale=cfg["sm_scale"],
                       device=DEV, **kw)


def run_gpu(cfg: dict, v: mv.Verifier | None = None, dev_inputs: dict | None = None, **kw):
    v = v or verifier_for(cfg, **kw)
    d = dev_inputs or upload(cfg)
    out, lse = v.run(d["q"], d["pool"], d["kv_indices"], d["prefix_lens"], d["tree_parent"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), v


def run_oracle(cfg: dict, nodes=None):
    return orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"], cfg["tree_parent"],
                                cfg["sm_scale"], nodes=nodes)


def compare(out, lse, ref_out, ref_lse, *, rows=None, strict=True, lse_abs=LSE_ABS_STRICT):
    """Assert GPU (out, lse) against the oracle on the rows where the oracle was evaluated."""
    if rows is None:
        rows = ~np.isnan(ref_lse)
    o, ro = out[rows], ref_out[rows]
    l, rl = lse[rows], ref_lse[rows]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), "non-finite GPU output"
    d = np.abs(o - ro)
    bad = d > OUT_ATOL + OUT_RTOL * np.abs(ro)
    assert not bad.any(), f"out outside contract tolerance: max |d| {d.max():.3e}"
    dl = np.abs(l - rl)
    assert dl.max() <= LSE_ATOL, f"lse outside contract tolerance: {dl.max():.3e}"
    rel = np.linalg.norm(o - ro, axis=-1) / np.maximum(np.linalg.norm(ro, axis=-1), 1e-30)
    if strict:
        assert rel.max() <= ROW_REL_L2, f"row relative L2 error {rel.max():.3e}"
        assert dl.max() <= lse_abs, f"lse error {dl.max():.3e}"
    return dict(max_abs_out=float(d.max()), max_row_rel=float(rel.max()), max_abs_lse=float(dl.max()))
