"""GPU parity of Tier-1 relocation (mlaverify_relocate) against its CPU oracle, through the C ABI.

Relocation is byte work, so the bar is bit-exact: the pool rows, the rewritten index
list and the refusal bits must equal the oracle's.  The verify pass must give
bit-identical results before and after a relocation (it only permutes pool slots).
"""

import numpy as np
import pytest
import torch

import mla_tree_verify_mlaverify_amd as mv
from gpu_util import DEV, bf16, i32, run_gpu, upload, verifier_for
from oracle import relocate_oracle as rel
from workloads import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def pool_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def relocate_gpu(cfg, v, d, dst, max_prefix=None):
    dst_t = i32(dst)
    v.relocate(d["pool"], d["kv_indices"], d["prefix_lens"], dst_t, cfg["tree_nodes"])
    torch.cuda.synchronize()
    return v.read_device_errors()


CASES = [
    # seed, prefix per request, T, slots, row stride
    (0, [40, 0, 17], 5, 512, 576),
    (1, [1], 1, 64, 576),
    (2, [64, 65, 31, 33], 9, 1024, 576),
    (3, [300, 1000], 16, 4096, 640),
    (4, [5] * 100, 2, 2048, 576),
]


@pytest.mark.parametrize("seed,prefix,t,slots,stride", CASES)
def test_relocation_matches_oracle_bit_exact(seed, prefix, t, slots, stride):
    cfg = synth.defrag_config(seed, batch=len(prefix), prefix=prefix, tree_nodes=t, heads=2, slots=slots,
                              row_stride=stride)
    v = verifier_for(cfg, max_prefix=max(prefix) + 3)
    d = upload(cfg)
    err = relocate_gpu(cfg, v, d, cfg["dst_start"])
    pool, idx, rerr = rel.relocate(cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"], t, cfg["dst_start"],
                                   max(prefix) + 3)
    assert err == rerr == 0
    assert np.array_equal(d["kv_indices"].cpu().numpy(), idx)
    assert np.array_equal(pool_bits(d["pool"]), pool)


def test_verify_output_unchanged_and_fast_path_applies():
    cfg = synth.defrag_config(5, batch=3, prefix=[700, 64, 1500], tree_nodes=12, heads=8, slots=8192)
    v = verifier_for(cfg)
    d = upload(cfg)
    a, la, _ = run_gpu(cfg, v, d)
    assert relocate_gpu(cfg, v, d, cfg["dst_start"]) == 0
    b, lb, _ = run_gpu(cfg, v, d)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    # the prefixes are now runs: the contiguous-run path gives the same bits as row gathers
    v2 = verifier_for(cfg, flags=mv.FLAG_NO_FASTPATH)
    c, lc, _ = run_gpu(cfg, v2, d)
    assert np.array_equal(b, c) and np.array_equal(lb, lc)


def test_second_relocation_and_in_place_call():
    cfg = synth.defrag_config(6, batch=2, prefix=[200, 120], tree_nodes=4, heads=1, slots=2048)
    v = verifier_for(cfg)
    d = upload(cfg)
    assert relocate_gpu(cfg, v, d, cfg["dst_start"]) == 0
    pool1, idx1 = pool_bits(d["pool"]).copy(), d["kv_indices"].cpu().numpy().copy()
    # the same call again: every row already sits at its destination, nothing changes
    assert relocate_gpu(cfg, v, d, cfg["dst_start"]) == 0
    assert np.array_equal(pool_bits(d["pool"]), pool1) and np.array_equal(d["kv_indices"].cpu().numpy(), idx1)
    # run to run: move request 0 into the free lower slots 0..199 only if they are free
    used = set(idx1.tolist())
    free0 = next(s for s in range(0, 1024 - 200) if not any((s + j) in used for j in range(200)))
    dst2 = np.array([free0, -1], dtype=np.int32)
    pool, idx, rerr = rel.relocate(pool1, idx1, cfg["prefix_lens"], 4, dst2, 200)
    assert relocate_gpu(cfg, v, d, dst2) == rerr == 0
    assert np.array_equal(d["kv_indices"].cpu().numpy(), idx)
    assert np.array_equal(pool_bits(d["pool"]), pool)


def tiny_inputs():
    pool = np.repeat(np.arange(16, dtype=np.uint16)[:, None], 576, axis=1)
    idx = np.array([3, 1, 7, 0, 5, 2, 9], dtype=np.int32)
    return pool, idx


@pytest.mark.parametrize("dst,plens,idx_patch", [
    ([10, -1], [3, 2], None),
    ([10, 13], [3, 2], None),
    ([4, -1], [3, 2], None),
    ([-1, 8], [3, 2], None),
    ([-1, 6], [3, 2], None),
    ([10, 11], [3, 2], None),
    ([14, -1], [3, 2], None),
    ([10, -1], [3, 17], None),
    ([10, -1], [-1, 2], None),
    ([10, -1], [3, 2], (6, 16)),
    ([10, 4], [3, 2], (6, -3)),
    ([4, -1], [3, 2], [4, 1, 12, 0, 13, 2, 9]),  # request 0 partly in place: 4 stays, 1 -> 5, 12 -> 6
    ([4, -1], [3, 2], [5, 4, 6, 0, 13, 2, 9]),   # 4 and 5 swap places: a conflict
])
def test_refusals_and_small_cases_match_oracle(dst, plens, idx_patch):
    pool, idx = tiny_inputs()
    if isinstance(idx_patch, tuple):
        idx[idx_patch[0]] = idx_patch[1]
    elif idx_patch is not None:
        idx = np.array(idx_patch, dtype=np.int32)
    v = mv.Verifier(num_heads=1, max_batch=2, max_tree_nodes=1, max_prefix_len=16, pool_slots=16, device=DEV)
    v.read_device_errors()
    d_pool = torch.from_numpy(pool.view(np.int16)).view(torch.bfloat16).to(DEV)
    d_idx = i32(idx)
    # segment offsets of a bad prefix length would run past the index list: give it room
    d_idx_room = torch.full((64,), -7, dtype=torch.int32, device=DEV)
    d_idx_room[:len(idx)] = d_idx
    v.relocate(d_pool, d_idx_room, i32(plens), i32(dst), 1)
    torch.cuda.synchronize()
    err = v.read_device_errors()
    rpool, ridx, rerr = rel.relocate(pool, idx, plens, 1, dst, 16)
    assert err == rerr
    assert np.array_equal(pool_bits(d_pool), rpool)
    assert np.array_equal(d_idx_room.cpu().numpy()[:len(idx)], ridx)


def test_full_size_relocation_sampled():
    """The benchmark's relocation: a 185,000-token prefix scattered over the lower half of a
    524,288-slot pool moves to a run in the upper half.  Every index is compared; pool rows
    are compared on a sample of destinations and on untouched rows."""
    rng = np.random.default_rng(77)
    slots, p, t = 524288, 185000, 64
    pool = rng.integers(0, 1 << 16, size=(slots, 576), dtype=np.uint16)  # any bits: the copy is bytewise
    idx = rng.choice(slots // 2, size=p + t, replace=False).astype(np.int32)
    dst = np.array([slots // 2 + 12345], dtype=np.int32)
    v = mv.Verifier(num_heads=8, max_batch=1, max_tree_nodes=t, max_prefix_len=p, pool_slots=slots, device=DEV)
    d_pool = torch.from_numpy(pool.view(np.int16)).view(torch.bfloat16).to(DEV)
    d_idx = i32(idx)
    v.relocate(d_pool, d_idx, i32([p]), i32(dst), t)
    torch.cuda.synchronize()
    assert v.read_device_errors() == 0
    got_idx = d_idx.cpu().numpy()
    assert np.array_equal(got_idx[:p], np.arange(dst[0], dst[0] + p)) and np.array_equal(got_idx[p:], idx[p:])
    got = d_pool.view(torch.int16)
    js = np.concatenate([[0, p - 1], rng.integers(0, p, 2000)])
    rows = torch.from_numpy(dst[0] + js).to(DEV)
    assert np.array_equal(got[rows].cpu().numpy().view(np.uint16), pool[idx[js]])
    untouched = np.concatenate([idx[:100], rng.integers(0, slots // 2, 1000), [slots - 1]])
    rows = torch.from_numpy(untouched).to(DEV)
    assert np.array_equal(got[rows].cpu().numpy().view(np.uint16), pool[untouched])
