"""The allocation-free verify entry point (mlaverify_run_static, for callers that cannot
allocate) against the handle-based mlaverify_run, through the C ABI: the same kernels over a
static device workspace must give the same bits.  Two calls in a row, the second smaller,
show that nothing left in the shared static array from one call leaks into the next."""

import numpy as np
import pytest
import torch

import mla_tree_verify_mlaverify_amd as mv
from gpu_util import DEV, compare, run_gpu, run_oracle, upload
from workloads import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def lib_config(cfg, **kw):
    return mv.make_config(cfg["heads"], cfg["batch"], cfg["tree_nodes"], max(1, int(cfg["prefix_lens"].max())),
                          cfg["slots"], cfg["row_stride"], cfg["sm_scale"], **kw)


def run_static(cfg, d, **kw):
    b, t, h = cfg["batch"], cfg["tree_nodes"], cfg["heads"]
    out = torch.full((b * t, h, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((b * t, h), float("nan"), dtype=torch.float32, device=DEV)
    mv.run_static(lib_config(cfg, **kw), d["q"], d["pool"], d["kv_indices"], d["prefix_lens"], d["tree_parent"],
                  out, lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def test_static_entry_matches_run_on_two_calls():
    first = synth.make_config(1)  # 4,096-token prefix, 64 nodes, 8 heads: 4 M tiles, 65 units
    second = synth.small_config(60, batch=3, prefix=[300, 45, 0], tree_nodes=9, heads=8, slots=4096,
                                tree="forest", q_scale=1.0)
    for cfg in (first, second):
        d = upload(cfg)
        a, la, _ = run_gpu(cfg, dev_inputs=d)
        b, lb = run_static(cfg, d)
        assert np.array_equal(a, b) and np.array_equal(la, lb)
        ref_out, ref_lse = run_oracle(cfg)
        compare(b, lb, ref_out, ref_lse)


def test_static_entry_fixed_split_and_no_fastpath():
    cfg = synth.make_config(1, variant="contiguous")
    d = upload(cfg)
    a, la, _ = run_gpu(cfg, dev_inputs=d, split_tokens=256, flags=mv.FLAG_NO_FASTPATH)
    b, lb = run_static(cfg, d, split_tokens=256, flags=mv.FLAG_NO_FASTPATH)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_static_entry_refuses_calls_beyond_its_workspace():
    # 128 heads x 256 nodes: 256 M tiles of one unit each, 2 x 32,768 rows of partials (67 MB)
    cfg = synth.small_config(61, batch=1, prefix=[40], tree_nodes=256, heads=128, slots=1024, q_scale=1.0)
    d = upload(cfg)
    out = torch.full((256, 128, 512), 3.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((256, 128), 3.0, dtype=torch.float32, device=DEV)
    with pytest.raises(mv.MlaVerifyError) as e:
        mv.run_static(lib_config(cfg), d["q"], d["pool"], d["kv_indices"], d["prefix_lens"], d["tree_parent"], out,
                      lse)
    assert e.value.status == mv.binding.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out.float() == 3.0) and torch.all(lse == 3.0)
