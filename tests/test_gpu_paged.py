"""GPU parity of paged prefixes (a block table of page ids, page_size > 1) through the C ABI.

A paged batch must give the same bits as the same batch described token by token (its
expansion by the oracle's expand_block_table, run with page_size 1): the keys, their order
and the work partition are the same.  Results are also checked against the fp64 oracle.
"""

import numpy as np
import pytest
import torch

import mla_tree_verify_mlaverify_amd as mv
from gpu_util import DEV, compare, i32, run_gpu, upload, verifier_for
from oracle import mla_tree_oracle as orc
from workloads import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

PAGED = [
    # seed, prefix per request, T, H, pool slots, page size, fixed split (0: automatic)
    (0, [37, 70], 5, 8, 4096, 16, 0),
    (1, [1000], 64, 8, 8192, 64, 0),
    (2, [300, 0, 513], 9, 4, 8192, 2, 96),
    (3, [4097], 17, 16, 16384, 256, 0),
    (4, [2000, 33], 8, 8, 32768, 1024, 0),
    (5, [640], 33, 8, 4096, 32, 64),
    (6, [129], 3, 2, 4096, 8, 32),
    # one M tile of 65..128 rows (gathers staged in VGPRs), also with a big tree
    (7, [1500, 300], 16, 8, 16384, 16, 0),
    (8, [700], 100, 1, 8192, 32, 0),
]


def expanded(cfg):
    flat = dict(cfg)
    flat["kv_indices"] = orc.expand_block_table(cfg["kv_indices"], cfg["prefix_lens"], cfg["tree_nodes"],
                                                cfg["page_size"]).astype(np.int32)
    return flat


@pytest.mark.parametrize("seed,prefix,t,h,slots,page,split", PAGED)
def test_paged_equals_its_expansion_and_oracle(seed, prefix, t, h, slots, page, split):
    cfg = synth.paged_config(seed, batch=len(prefix), prefix=prefix, tree_nodes=t, heads=h, slots=slots, page=page)
    flat = expanded(cfg)
    a, la, v = run_gpu(cfg, page_size=page, split_tokens=split)
    b, lb, _ = run_gpu(flat, split_tokens=split)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    assert v.read_device_errors() == 0
    ref_out, ref_lse = orc.verify_attention(flat["q"], flat["pool"], flat["kv_indices"], flat["prefix_lens"],
                                            flat["tree_parent"], flat["sm_scale"])
    compare(a, la, ref_out, ref_lse)


def test_paged_reference_raise_on_the_helper_path():
    # 64 rows in one M tile (the helper-wave path), fixed 256-token units, and in each request
    # a dominant key at prefix position 100: the fourth tile of the first unit raises every
    # row's reference, so each row's accumulator and sum are rescaled once mid-unit while the
    # helper waves keep gathering through the block table
    cfg = synth.paged_config(9, batch=2, prefix=[1500, 700], tree_nodes=8, heads=8, slots=16384, page=16)
    flat = expanded(cfg)
    u = np.where(np.random.default_rng(9).integers(0, 2, size=synth.LATENT_DIM) == 1, 1.0, -1.0).astype(np.float32)
    pool = cfg["pool"].copy()
    for off in synth.request_offsets(cfg["prefix_lens"], cfg["tree_nodes"]):
        pool[int(flat["kv_indices"][off + 100]), :synth.LATENT_DIM] = synth.f32_to_bf16_bits(2.0 * u)
    q = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(cfg["q"]) + 0.5 * u[None, None, :])
    cfg = dict(cfg, pool=pool, q=q)
    flat = dict(flat, pool=pool, q=q)
    a, la, v = run_gpu(cfg, page_size=16, split_tokens=256)
    b, lb, _ = run_gpu(flat, split_tokens=256)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    assert v.read_device_errors() == 0 and v.read_plan()["n_mtiles"] == 1
    ref_out, ref_lse = orc.verify_attention(flat["q"], flat["pool"], flat["kv_indices"], flat["prefix_lens"],
                                            flat["tree_parent"], flat["sm_scale"])
    compare(a, la, ref_out, ref_lse)
    assert np.abs(ref_out).max() > 1.0  # the needle dominates


def test_consecutive_pages_take_the_fast_path():
    cfg = synth.paged_config(7, batch=2, prefix=[900, 260], tree_nodes=12, heads=8, slots=8192, page=64,
                             contiguous_pages=True)
    a, la, _ = run_gpu(cfg, page_size=64)
    b, lb, _ = run_gpu(cfg, page_size=64, flags=mv.FLAG_NO_FASTPATH)
    c, lc, _ = run_gpu(expanded(cfg))
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    assert np.array_equal(a, c) and np.array_equal(la, lc)


@pytest.mark.parametrize("page,slots,bad_entry", [
    (16, 4096, 256),       # first page id past the pool
    (1024, 32768, 1 << 22),  # shifted by the page size this would wrap to slot 0
    (8, 4096, -1),
])
def test_page_ids_outside_the_pool_poison_their_request(page, slots, bad_entry):
    cfg = synth.paged_config(8, batch=2, prefix=[100, 300], tree_nodes=4, heads=4, slots=slots, page=page)
    bad = dict(cfg)
    idx = cfg["kv_indices"].copy()
    first_page_req1 = -(-100 // page) + 4  # request 0's pages, its 4 tree slots
    idx[first_page_req1] = bad_entry
    bad["kv_indices"] = idx
    out, lse, v = run_gpu(bad, page_size=page)
    assert v.read_device_errors() == mv.DEVERR_BAD_INDEX
    assert np.all(np.isnan(out[4:])) and np.all(np.isnan(lse[4:]))
    ref_out, ref_lse = orc.verify_attention(cfg["q"], cfg["pool"], expanded(cfg)["kv_indices"], cfg["prefix_lens"],
                                            cfg["tree_parent"], cfg["sm_scale"])
    compare(out[:4], lse[:4], ref_out[:4], ref_lse[:4])


def test_relocation_needs_single_token_slots():
    cfg = synth.paged_config(9, batch=1, prefix=[64], tree_nodes=2, heads=1, slots=1024, page=16)
    v = verifier_for(cfg, page_size=16)
    d = upload(cfg)
    with pytest.raises(mv.MlaVerifyError):
        v.relocate(d["pool"], d["kv_indices"], d["prefix_lens"], i32([512]), 2)
