"""Pins of the relocation oracle (oracle/relocate_oracle.py) on the CPU.

The expected values do not come from the oracle's own rules: a relocation permutes
pool slots, so the verify attention (its own oracle, pinned in test_oracle.py) must
not change at all; the relocated prefixes must be the runs asked for; and each
refusal case below is derived by hand from the stated contract.
"""

import math

import numpy as np
import pytest

from oracle import mla_tree_oracle as orc
from oracle import relocate_oracle as rel
from workloads import synth

SCALE = 1.0 / math.sqrt(192.0)


def attention(cfg, pool, idx):
    return orc.verify_attention(cfg["q"], pool, idx, cfg["prefix_lens"], cfg["tree_parent"], SCALE)


@pytest.mark.parametrize("seed,prefix,t", [(0, [40, 0, 17], 5), (1, [1], 1), (2, [64, 65], 9)])
def test_relocation_preserves_attention_and_makes_runs(seed, prefix, t):
    cfg = synth.defrag_config(seed, batch=len(prefix), prefix=prefix, tree_nodes=t, heads=2, slots=512)
    pool, idx, err = rel.relocate(cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"], t, cfg["dst_start"], 1000)
    assert err == 0
    a = attention(cfg, cfg["pool"], cfg["kv_indices"])
    b = attention(cfg, pool, idx)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    off = 0
    moved = np.zeros(512, dtype=bool)
    for r, p in enumerate(prefix):
        if p:
            d = int(cfg["dst_start"][r])
            assert np.array_equal(idx[off:off + p], np.arange(d, d + p))
            moved[d:d + p] = True
        assert np.array_equal(idx[off + p:off + p + t], cfg["kv_indices"][off + p:off + p + t])  # tree kept
        off += p + t
    assert np.array_equal(pool[~moved], cfg["pool"][~moved])  # nothing else is written


def test_skipped_request_is_untouched():
    cfg = synth.defrag_config(3, batch=2, prefix=[20, 30], tree_nodes=4, heads=1, slots=256)
    dst = cfg["dst_start"].copy()
    dst[0] = -1
    pool, idx, err = rel.relocate(cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"], 4, dst, 1000)
    assert err == 0
    assert np.array_equal(idx[:24], cfg["kv_indices"][:24])
    assert np.array_equal(idx[24:54], np.arange(dst[1], dst[1] + 30))


def tiny():
    """Pool of 16 rows (row r filled with r); request 0: prefix slots 3, 1, 7 and tree slot 0;
    request 1: prefix slots 5, 2 and tree slot 9."""
    pool = np.repeat(np.arange(16, dtype=np.uint16)[:, None], 576, axis=1)
    idx = np.array([3, 1, 7, 0, 5, 2, 9], dtype=np.int32)
    return pool, idx, [3, 2]


@pytest.mark.parametrize("dst,plens,idx_patch,expect", [
    ([10, -1], None, None, 0),                          # free run 10..12
    ([10, 13], None, None, 0),                          # two adjacent free runs
    ([4, -1], None, None, rel.ERR_CONFLICT),            # 5 is request 1's prefix slot
    ([-1, 8], None, None, rel.ERR_CONFLICT),            # 9 is request 1's own tree slot
    ([-1, 6], None, None, rel.ERR_CONFLICT),            # 7 is request 0's prefix slot
    ([10, 11], None, None, rel.ERR_CONFLICT),           # runs 10..12 and 11..12 overlap
    ([14, -1], None, None, rel.ERR_CONFLICT),           # 14..16 leaves the 16-row pool
    ([10, -1], [3, 17], None, rel.ERR_BAD_PREFIX),      # P_1 = 17 > max_prefix = 16
    ([10, -1], [-1, 2], None, rel.ERR_BAD_PREFIX),
    ([10, -1], None, (6, 16), rel.ERR_BAD_INDEX),       # tree slot 16 is outside the pool
    ([10, 4], None, (6, -3), rel.ERR_BAD_INDEX | rel.ERR_CONFLICT),  # and 5 is in use
])
def test_refusals_leave_everything_untouched(dst, plens, idx_patch, expect):
    pool, idx, p = tiny()
    if plens is not None:
        p = plens
    if idx_patch is not None:
        idx = idx.copy()
        idx[idx_patch[0]] = idx_patch[1]
    new_pool, new_idx, err = rel.relocate(pool, idx, p, 1, dst, 16)
    assert err == expect
    if expect:
        assert np.array_equal(new_pool, pool) and np.array_equal(new_idx, idx)
    else:
        assert new_pool[10, 0] == 3 and new_pool[11, 0] == 1 and new_pool[12, 0] == 7
        assert new_idx[:3].tolist() == [10, 11, 12] and new_idx[3] == 0


def test_rows_already_in_place_are_allowed():
    pool, idx, p = tiny()
    idx = np.array([4, 5, 6, 0, 12, 2, 9], dtype=np.int32)  # request 0 already sits at 4..6
    new_pool, new_idx, err = rel.relocate(pool, idx, p, 1, [4, -1], 16)
    assert err == 0 and np.array_equal(new_pool, pool) and np.array_equal(new_idx, idx)
    # partly in place: 4 and 5 stay, slot 12 moves to 6
    idx2 = np.array([4, 5, 12, 0, 13, 2, 9], dtype=np.int32)
    new_pool, new_idx, err = rel.relocate(pool, idx2, p, 1, [4, -1], 16)
    assert err == 0 and new_idx[:3].tolist() == [4, 5, 6] and new_pool[6, 0] == 12
    # a row in place at the wrong position is still a conflict (5 would be overwritten first)
    idx3 = np.array([5, 4, 6, 0, 13, 2, 9], dtype=np.int32)
    assert rel.relocate(pool, idx3, p, 1, [4, -1], 16)[2] == rel.ERR_CONFLICT


def test_duplicate_slots_are_separate_keys():
    pool, idx, p = tiny()
    idx = np.array([3, 3, 7, 0, 5, 2, 9], dtype=np.int32)
    new_pool, new_idx, err = rel.relocate(pool, idx, p, 1, [10, -1], 16)
    assert err == 0 and new_pool[10, 0] == 3 and new_pool[11, 0] == 3 and new_idx[:3].tolist() == [10, 11, 12]


def test_only_latent_columns_move():
    cfg = synth.defrag_config(4, batch=1, prefix=[8], tree_nodes=2, heads=1, slots=64, row_stride=640)
    pool, idx, err = rel.relocate(cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"], 2, cfg["dst_start"], 100)
    d = int(cfg["dst_start"][0])
    assert err == 0
    assert np.array_equal(pool[d:d + 8, 576:], cfg["pool"][d:d + 8, 576:])  # padding not copied
    assert np.array_equal(pool[d:d + 8, :576], cfg["pool"][cfg["kv_indices"][:8], :576])
