"""Pins of the CPU fp64 oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a hand-derived fixture, a closed
form, an identity of the mathematics, brute force, or a library routine that the
special case reduces to (torch's scaled_dot_product_attention in float64 on the
CPU).  None of these reuse the oracle's own ancestor walk or softmax code.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import mla_tree_oracle as orc
from workloads import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_tree.txt")
SCALE = 1.0 / math.sqrt(192.0)


def read_golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = [int(x, 0) for x in rest]
    return vals


def closure_masks(parents):
    """Ancestor-or-self sets by transitive closure of the child->parent relation.

    reach starts as I + A (A[i, p] = 1 when p is i's parent) and is squared until it
    stops changing; a different algorithm from walking parent pointers.
    """
    t = len(parents)
    reach = np.eye(t, dtype=np.int64)
    for i, p in enumerate(parents):
        if p >= 0:
            reach[i, p] = 1
    while True:
        nxt = np.minimum(reach @ reach, 1)
        if np.array_equal(nxt, reach):
            break
        reach = nxt
    return reach.astype(bool)  # reach[i, j]: j is i or an ancestor of i


def widen_f32(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def sdpa_reference(cfg, visible):
    """Per-request SDPA in float64 with an explicit boolean mask over [prefix ++ tree] keys.

    ``visible(b)`` returns the [T, T] tree visibility matrix of request b.
    """
    t, h = cfg["tree_nodes"], cfg["heads"]
    outs = []
    off = 0
    for b in range(cfg["batch"]):
        p = int(cfg["prefix_lens"][b])
        seg = cfg["kv_indices"][off:off + p + t]
        off += p + t
        keys = torch.from_numpy(widen_f32(cfg["pool"][seg, :576]))  # [P+T, 576]
        qb = torch.from_numpy(widen_f32(cfg["q"][b * t:(b + 1) * t]))  # [T, H, 576]
        mask = torch.zeros(t, p + t, dtype=torch.bool)
        mask[:, :p] = True
        mask[:, p:] = torch.from_numpy(visible(b))
        qh = qb.permute(1, 0, 2).unsqueeze(0)  # [1, H, T, 576]
        k = keys.unsqueeze(0).unsqueeze(0).expand(1, h, p + t, 576)
        v = keys[:, :512].unsqueeze(0).unsqueeze(0).expand(1, h, p + t, 512)
        o = torch.nn.functional.scaled_dot_product_attention(
            qh, k, v, attn_mask=mask.unsqueeze(0).unsqueeze(0), scale=SCALE)
        outs.append(o[0].permute(1, 0, 2).numpy())  # [T, H, 512]
    return np.concatenate(outs, axis=0)


# --------------------------------------------------------------------------- masks

def test_tiny_masks_match_hand_derivation():
    g = read_golden()
    masks = orc.ancestor_masks(np.array(g["parents"]))
    assert [int(m) for m in masks] == g["masks"]
    slots = [len(orc.visible_slots(np.arange(264), np.array([256]), np.array([g["parents"]]), 0, i))
             for i in range(8)]
    assert slots == g["visible"]
    assert list(synth.tree_depths(g["parents"])) == g["depth"]


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("kind", ["random", "chain", "forest"])
def test_masks_match_transitive_closure(seed, kind):
    rng = np.random.default_rng(seed)
    t = int(rng.integers(1, 65))
    if kind == "random":
        parents = synth.random_tree(rng, t)
    elif kind == "chain":
        parents = synth.chain_tree(t)
    else:
        parents = np.array([int(rng.integers(-1, i)) for i in range(t)], dtype=np.int32)
    masks = orc.ancestor_masks(parents)
    reach = closure_masks(parents)
    for i in range(t):
        bits = [(int(masks[i]) >> j) & 1 for j in range(t)]
        assert bits == reach[i].astype(int).tolist()
        assert int(masks[i]) >> t == 0


@pytest.mark.parametrize("t,kind", [(65, "chain"), (100, "random"), (128, "forest"), (200, "random"),
                                    (256, "chain"), (256, "forest")])
def test_mask_words_match_transitive_closure(t, kind):
    rng = np.random.default_rng(t)
    if kind == "random":
        parents = synth.random_tree(rng, t)
    elif kind == "chain":
        parents = synth.chain_tree(t)
    else:
        parents = np.array([int(rng.integers(-1, i)) for i in range(t)], dtype=np.int32)
    words = orc.ancestor_mask_words(parents)
    assert words.shape == (t, -(-t // 64))
    reach = closure_masks(parents)
    for i in range(t):
        bits = [(int(words[i, j // 64]) >> (j % 64)) & 1 for j in range(64 * words.shape[1])]
        assert bits[:t] == reach[i].astype(int).tolist() and not any(bits[t:])


def test_invalid_parent_rejected():
    with pytest.raises(ValueError):
        orc.ancestor_masks(np.array([-1, 0, 2]))  # node 2 is its own parent
    with pytest.raises(ValueError):
        orc.ancestor_masks(np.array([0]))  # root must be -1
    with pytest.raises(ValueError):
        orc.ancestor_masks(np.array([-1, -2]))


def test_random_tree_depth_bound():
    rng = np.random.default_rng(7)
    for _ in range(50):
        parents = synth.random_tree(rng, 64)
        assert parents[0] == -1
        assert all(-1 <= p < i for i, p in enumerate(parents))
        assert synth.tree_depths(parents).max() <= 8


# --------------------------------------------------------------------------- inputs

def test_bf16_widening_known_values():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0xFF80, 0x3E4D, 0x0000, 0x8000], dtype=np.uint16)
    v = orc.bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0
    assert v[2] == 2.0 ** -133  # smallest bf16 subnormal
    assert v[3] == math.inf and v[4] == -math.inf
    assert v[5] == 0.2001953125  # 0x3E4D = 1.6015625 * 2^-3
    assert v[6] == 0.0 and math.copysign(1.0, v[7]) == -1.0
    assert np.isnan(orc.bf16_to_f64(np.array([0x7FC0], dtype=np.uint16)))[0]


def test_f32_to_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -2.5,
                  3.0e38, np.inf, np.nan], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    assert b[0] == 0x3F80
    assert b[1] == 0x3F80  # tie -> even
    assert b[2] == 0x3F82  # tie -> even (up)
    assert b[3] == 0x3F81  # above the tie -> up
    assert b[4] == 0xC020
    assert b[5] == 0x7F62  # 3e38 rounds within range
    assert b[6] == 0x7F80
    assert (b[7] & 0x7F80) == 0x7F80 and (b[7] & 0x007F) != 0


def test_f32_to_bf16_extremes_and_nearest():
    x = np.array([3.4028235e38, -3.4028235e38, -np.inf, 1e-45, -1e-45, 0.0, -0.0], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    assert b.tolist() == [0x7F80, 0xFF80, 0xFF80, 0x0000, 0x8000, 0x0000, 0x8000]
    n = synth.f32_to_bf16_bits(np.array([-np.nan], dtype=np.float32))[0]
    assert (n & 0x8000) and (n & 0x7F80) == 0x7F80 and (n & 0x7F)
    # every finite result is a nearest bf16 value (checked against both neighbours), ties to even
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-80, 80, 200000))).astype(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.0e38)]
    b = synth.f32_to_bf16_bits(x).astype(np.int64)
    got = orc.bf16_to_f64(b.astype(np.uint16))
    xd = x.astype(np.float64)
    for nb in (b - 1, b + 1):
        ok = (nb & 0x7F80) != 0x7F80  # neighbours that are finite bf16 patterns
        other = orc.bf16_to_f64((nb & 0xFFFF).astype(np.uint16))
        d, dn = np.abs(xd - got), np.abs(xd - other)
        assert np.all(~ok | (np.sign(other) != np.sign(got)) | (d < dn) | ((d == dn) & (b % 2 == 0)))


def test_generator_is_deterministic_and_shaped():
    a = synth.make_config(0)
    b = synth.make_config(0)
    for k in ("q", "pool", "kv_indices", "prefix_lens", "tree_parent"):
        assert np.array_equal(a[k], b[k])
    assert a["q"].shape == (8, 8, 576) and a["pool"].shape == (512, 576)
    assert np.array_equal(a["kv_indices"], np.arange(264))
    assert a["tree_parent"].tolist() == [[-1, 0, 1, 2, 0, 4, 1, 6]]
    c = synth.make_config(1)
    assert len(np.unique(c["kv_indices"])) == len(c["kv_indices"]) == 4096 + 64
    assert c["kv_indices"].max() < 262144
    std = synth.bf16_bits_to_f32(c["q"]).std()
    assert 0.09 < std < 0.11


def test_batch_prefix_lengths_log_uniform_range():
    rng_cfg = synth.CONFIGS[4]
    lo, hi = rng_cfg["prefix"][1], rng_cfg["prefix"][2]
    lens = synth._draw_prefix_lens(np.random.default_rng(0), rng_cfg["prefix"], 4000)
    assert lens.min() >= lo and lens.max() <= hi
    # log-uniform: the median of log-length sits at the midpoint of [ln lo, ln hi]
    mid = 0.5 * (math.log(lo) + math.log(hi))
    assert abs(np.median(np.log(lens)) - mid) < 0.15


# --------------------------------------------------------------------------- closed forms

def test_q_zero_closed_form_tiny():
    """q = 0: every score is 0, so lse = ln(#visible) and out = plain mean of the visible V rows."""
    g = read_golden()
    cfg = synth.make_config(0, variant="qzero")
    out, lse = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                                    cfg["tree_parent"], SCALE)
    v = widen_f32(cfg["pool"][:, :512])
    for i in range(8):
        rows = list(range(256)) + [256 + j for j in range(8) if (g["masks"][i] >> j) & 1]
        assert len(rows) == g["visible"][i]
        np.testing.assert_allclose(lse[i], math.log(g["visible"][i]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(out[i], np.broadcast_to(v[rows].mean(axis=0), (8, 512)),
                                   rtol=0, atol=1e-14)
    # printed values in the fixture
    assert abs(lse[0, 0] - 5.5490760848952201) < 1e-13
    assert abs(lse[3, 0] - 5.5606816310155276) < 1e-13


def test_constant_keys_closed_form():
    """Every pool row equal to k: out = k[:512] and lse = sigma*q.k + ln(#visible)."""
    cfg = synth.small_config(3, batch=2, prefix=[5, 0], tree_nodes=6, heads=3, slots=64)
    k = cfg["pool"][7].copy()
    cfg["pool"] = np.broadcast_to(k, cfg["pool"].shape).copy()
    out, lse = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                                    cfg["tree_parent"], SCALE)
    kf = [float(x) for x in widen_f32(k)]
    for b in range(2):
        reach = closure_masks(cfg["tree_parent"][b])
        for i in range(6):
            count = int(cfg["prefix_lens"][b]) + int(reach[i].sum())
            for hh in range(3):
                qv = [float(x) for x in widen_f32(cfg["q"][b * 6 + i, hh])]
                dot = math.fsum(a * c for a, c in zip(qv, kf))
                assert abs(lse[b * 6 + i, hh] - (SCALE * dot + math.log(count))) < 1e-12
                np.testing.assert_allclose(out[b * 6 + i, hh], kf[:512], rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------- brute force / library

@pytest.mark.parametrize("seed,prefix,tree", [
    (0, [17, 3], "random"), (1, [0, 9], "forest"), (2, [11], "chain"), (3, [4, 0, 6], "random"),
])
def test_matches_brute_force(seed, prefix, tree):
    cfg = synth.small_config(seed, batch=len(prefix), prefix=prefix, tree_nodes=5, heads=2,
                             slots=96, tree=tree, q_scale=2.0)
    out, lse = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                                    cfg["tree_parent"], SCALE)
    bout, blse = orc.brute_force_verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"],
                                                  cfg["prefix_lens"], cfg["tree_parent"], SCALE)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, bout, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("seed,tree,t", [(0, "random", 8), (1, "random", 64), (2, "forest", 13),
                                         (3, "chain", 9)])
def test_matches_torch_sdpa_float64(seed, tree, t):
    cfg = synth.small_config(seed, batch=2, prefix=[40, 3], tree_nodes=t, heads=4, slots=4096,
                             tree=tree, q_scale=1.0)
    out, _ = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                                  cfg["tree_parent"], SCALE)
    ref = sdpa_reference(cfg, lambda b: closure_masks(cfg["tree_parent"][b]))
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-13)


def test_tiny_workload_matches_sdpa():
    cfg = synth.make_config(0)
    out, _ = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                                  cfg["tree_parent"], SCALE)
    g = read_golden()
    vis = np.array([[(m >> j) & 1 for j in range(8)] for m in g["masks"]], dtype=bool)
    ref = sdpa_reference(cfg, lambda b: vis)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-13)


def test_chain_tree_equals_causal_attention():
    """A chain tree is causal attention over prefix ++ tree, read off the last T rows."""
    cfg = synth.small_config(5, batch=1, prefix=[30], tree_nodes=12, heads=2, slots=1024,
                             tree="chain", q_scale=1.0)
    out, _ = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                                  cfg["tree_parent"], SCALE)
    p, t = 30, 12
    keys = torch.from_numpy(widen_f32(cfg["pool"][cfg["kv_indices"], :576]))
    qfull = torch.zeros(2, p + t, 576, dtype=torch.float64)
    qfull[:, p:] = torch.from_numpy(widen_f32(cfg["q"])).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(
        qfull.unsqueeze(0), keys.expand(1, 2, p + t, 576), keys[:, :512].expand(1, 2, p + t, 512),
        is_causal=True, scale=SCALE)
    ref = o[0, :, p:].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-13)


def test_single_node_is_plain_decode():
    """T = 1: the node sees the whole prefix and itself, i.e. unmasked attention over P+1 keys."""
    cfg = synth.small_config(6, batch=3, prefix=[50, 0, 7], tree_nodes=1, heads=5, slots=512,
                             q_scale=1.0)
    out, lse = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                                    cfg["tree_parent"], SCALE)
    off = 0
    for b, p in enumerate(cfg["prefix_lens"]):
        keys = torch.from_numpy(widen_f32(cfg["pool"][cfg["kv_indices"][off:off + p + 1], :576]))
        off += p + 1
        qb = torch.from_numpy(widen_f32(cfg["q"][b])).unsqueeze(1)  # [H, 1, 576]
        o = torch.nn.functional.scaled_dot_product_attention(
            qb, keys.expand(5, p + 1, 576), keys[:, :512].expand(5, p + 1, 512), scale=SCALE)
        np.testing.assert_allclose(out[b], o[:, 0].numpy(), rtol=1e-11, atol=1e-13)
    assert np.all(np.isfinite(lse))


# --------------------------------------------------------------------------- identities

def test_permuted_pool_gives_identical_result():
    cfg = synth.small_config(8, batch=2, prefix=[33, 21], tree_nodes=9, heads=3, slots=256)
    perm = synth.permute_pool(cfg, np.random.default_rng(99))
    a = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                             cfg["tree_parent"], SCALE)
    b = orc.verify_attention(perm["q"], perm["pool"], perm["kv_indices"], perm["prefix_lens"],
                             perm["tree_parent"], SCALE)
    assert not np.array_equal(cfg["kv_indices"], perm["kv_indices"])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_any_split_merged_by_lse_equals_single_pass():
    cfg = synth.small_config(9, batch=2, prefix=[70, 12], tree_nodes=7, heads=2, slots=512,
                             q_scale=1.5)
    out, lse = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                                    cfg["tree_parent"], SCALE)
    rng = np.random.default_rng(3)
    for b in range(2):
        for i in range(7):
            slots = orc.visible_slots(cfg["kv_indices"], cfg["prefix_lens"], cfg["tree_parent"], b, i)
            qrows = widen_f32(cfg["q"][b * 7 + i])
            cuts = np.sort(rng.integers(0, len(slots) + 1, size=4))
            parts = np.split(slots, cuts)  # may include empty parts
            outs, lses = zip(*[orc.attention_over_slots(qrows, cfg["pool"], s, SCALE) for s in parts])
            mo, ml = orc.lse_merge(outs, lses)
            np.testing.assert_allclose(ml, lse[b * 7 + i], rtol=0, atol=1e-12)
            np.testing.assert_allclose(mo, out[b * 7 + i], rtol=1e-12, atol=1e-14)


def test_merge_of_nothing_is_empty():
    o, l = orc.lse_merge([np.zeros((2, 512))] * 3, [np.full(2, -np.inf)] * 3)
    assert np.all(np.isneginf(l)) and np.all(o == 0)


def test_softmax_rows_sum_to_one():
    cfg = synth.small_config(10, batch=1, prefix=[100], tree_nodes=16, heads=4, slots=512, q_scale=3.0)
    for i in (0, 5, 15):
        w = orc.attention_weights(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                                  cfg["tree_parent"], SCALE, 0, i)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert np.all(w >= 0)


def test_attention_weights_reproduce_the_output():
    """The weights of Vis(b, i), applied to the visible V rows, give verify_attention's row (pinned
    against SDPA and brute force above), and the log of the weights of two keys differs by their
    score difference; with sharp queries a wrong scale or a dropped key fails both."""
    cfg = synth.small_config(13, batch=2, prefix=[50, 3], tree_nodes=6, heads=3, slots=512, q_scale=3.0)
    out, lse = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                                    cfg["tree_parent"], SCALE)
    for b in range(2):
        for i in range(6):
            w = orc.attention_weights(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                                      cfg["tree_parent"], SCALE, b, i)
            slots = orc.visible_slots(cfg["kv_indices"], cfg["prefix_lens"], cfg["tree_parent"], b, i)
            kv = orc.bf16_to_f64(cfg["pool"][slots, :576])
            np.testing.assert_allclose(w @ kv[:, :512], out[b * 6 + i], rtol=1e-12, atol=1e-14)
            s = SCALE * orc.bf16_to_f64(cfg["q"][b * 6 + i]) @ kv.T
            np.testing.assert_allclose(np.log(w[:, 1:]) - np.log(w[:, :1]), s[:, 1:] - s[:, :1], rtol=0, atol=1e-10)
            np.testing.assert_allclose(np.log(w), s - lse[b * 6 + i][:, None], rtol=0, atol=1e-10)


def test_prefix_order_invariance():
    cfg = synth.small_config(11, batch=2, prefix=[64, 31], tree_nodes=8, heads=2, slots=512)
    shuf = synth.permute_prefix(cfg, np.random.default_rng(5))
    a = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                             cfg["tree_parent"], SCALE)
    b = orc.verify_attention(shuf["q"], shuf["pool"], shuf["kv_indices"], shuf["prefix_lens"],
                             shuf["tree_parent"], SCALE)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-12)


def test_needle_dominates_where_visible():
    cfg = synth.small_config(12, batch=2, prefix=[40, 25], tree_nodes=10, heads=2, slots=512)
    cfg = synth.apply_variant(cfg, "needle_tree", np.random.default_rng(4))
    out, lse = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                                    cfg["tree_parent"], SCALE)
    for b in range(2):
        needle = widen_f32(cfg["pool"][cfg["needle_slots"][b], :512])
        reach = closure_masks(cfg["tree_parent"][b])
        for i in range(10):
            if reach[i, 1]:
                np.testing.assert_allclose(out[b * 10 + i], np.broadcast_to(needle, (2, 512)), atol=1e-6)
            else:
                assert np.abs(out[b * 10 + i]).max() < 0.5


def test_sharp_queries_still_match_brute_force():
    cfg = synth.small_config(13, batch=1, prefix=[20], tree_nodes=4, heads=2, slots=64, q_scale=3.0)
    out, lse = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                                    cfg["tree_parent"], SCALE)
    bout, blse = orc.brute_force_verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"],
                                                  cfg["prefix_lens"], cfg["tree_parent"], SCALE)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, bout, rtol=1e-12, atol=1e-14)


def test_column_scaling_commutes_exactly():
    """Scaling V column d by 2^k and q column d by 2^-k leaves every score unchanged, so
    the output column is scaled by exactly 2^k (all products and sums are exact shifts)."""
    cfg = synth.small_config(14, batch=2, prefix=[45, 70], tree_nodes=6, heads=3, slots=512)
    scaled = synth.apply_variant(cfg, "colscale")
    a = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"],
                             cfg["tree_parent"], SCALE)
    b = orc.verify_attention(scaled["q"], scaled["pool"], scaled["kv_indices"], scaled["prefix_lens"],
                             scaled["tree_parent"], SCALE)
    s = synth.column_scales()
    assert s.min() == 2.0 ** -12 and s.max() == 2.0 ** 12
    np.testing.assert_allclose(b[0] / s, a[0], rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(b[1], a[1], rtol=0, atol=1e-12)


def test_block_table_expansion_hand_derived():
    # page 4: request 0 (P=6) on pages 2, 0 -> slots 8..11, 0, 1; tree slot 30.
    # request 1 (P=3) on page 5 -> 20, 21, 22; tree slot 31.
    idx = np.array([2, 0, 30, 5, 31])
    got = orc.expand_block_table(idx, [6, 3], 1, 4)
    assert got.tolist() == [8, 9, 10, 11, 0, 1, 30, 20, 21, 22, 31]
    # page 1 leaves the list unchanged; P = 0 has no pages
    assert orc.expand_block_table(np.array([7, 3, 9, 1, 4]), [3, 0], 1, 1).tolist() == [7, 3, 9, 1, 4]
    assert orc.expand_block_table(np.array([9, 12]), [0, 0], 1, 64).tolist() == [9, 12]


def test_paged_layout_attention_equals_its_expansion():
    """The paged workload and its per-token expansion are the same attention (brute force on
    the expanded list)."""
    cfg = synth.paged_config(15, batch=2, prefix=[37, 70], tree_nodes=5, heads=2, slots=1024, page=16)
    flat = orc.expand_block_table(cfg["kv_indices"], cfg["prefix_lens"], 5, 16)
    assert len(flat) == 37 + 70 + 10 and len(set(flat.tolist())) == len(flat)
    out, lse = orc.verify_attention(cfg["q"], cfg["pool"], flat, cfg["prefix_lens"], cfg["tree_parent"], SCALE)
    bout, blse = orc.brute_force_verify_attention(cfg["q"], cfg["pool"], flat, cfg["prefix_lens"],
                                                  cfg["tree_parent"], SCALE)
    np.testing.assert_allclose(out, bout, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- ragged trees

def _ragged_case(seed, prefix, tree_lens, heads=2, slots=512, q_scale=1.0):
    """A packed batch with T_b = tree_lens[b]: every request drawn on its own from the
    workload recipe, then concatenated (rows, parents, index segments)."""
    parts = [synth.small_config(seed + 31 * b, batch=1, prefix=[p], tree_nodes=t, heads=heads, slots=slots,
                                tree="forest" if b % 2 else "random", q_scale=q_scale)
             for b, (p, t) in enumerate(zip(prefix, tree_lens))]
    pool = parts[0]["pool"]
    return dict(q=np.concatenate([c["q"] for c in parts]), pool=pool,
                kv_indices=np.concatenate([c["kv_indices"] for c in parts]),
                prefix_lens=np.array(prefix, dtype=np.int32), tree_lens=np.array(tree_lens, dtype=np.int32),
                tree_parent=np.concatenate([c["tree_parent"][0] for c in parts]), parts=parts)


def test_ragged_against_brute_force_per_request():
    case = _ragged_case(70, [5, 0, 9, 3], [1, 4, 3, 6])
    out, lse = orc.verify_attention_ragged(case["q"], case["pool"], case["kv_indices"], case["prefix_lens"],
                                           case["tree_lens"], case["tree_parent"], SCALE)
    n = 0
    off = 0
    for b, c in enumerate(case["parts"]):
        t, p = int(case["tree_lens"][b]), int(case["prefix_lens"][b])
        bo, bl = orc.brute_force_verify_attention(c["q"], case["pool"], case["kv_indices"][off:off + p + t],
                                                  [p], c["tree_parent"], SCALE)
        np.testing.assert_allclose(out[n:n + t], bo, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[n:n + t], bl, rtol=0, atol=1e-12)
        n += t
        off += p + t


def test_ragged_with_equal_trees_is_the_uniform_layout():
    cfg = synth.small_config(71, batch=3, prefix=[40, 7, 0], tree_nodes=5, heads=3, slots=512, q_scale=1.0)
    a = orc.verify_attention(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"], cfg["tree_parent"], SCALE)
    b = orc.verify_attention_ragged(cfg["q"], cfg["pool"], cfg["kv_indices"], cfg["prefix_lens"], [5, 5, 5],
                                    cfg["tree_parent"].reshape(-1), SCALE)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert orc.node_offsets([5, 5, 5]).tolist() == [0, 5, 10]
    assert orc.node_offsets([1, 64, 200, 3]).tolist() == [0, 1, 65, 265]


def test_ragged_matches_padding_with_extra_roots():
    # a 5-node tree padded to 9 nodes with extra roots (their own slots) gives the same rows
    case = _ragged_case(72, [30], [5])
    rng = np.random.default_rng(3)
    pad_slots = np.setdiff1d(np.arange(512), case["kv_indices"])[:4]
    q_pad = np.concatenate([case["q"], synth.f32_to_bf16_bits(rng.standard_normal((4, 2, 576), dtype=np.float32))])
    par_pad = np.concatenate([case["tree_parent"], [-1, -1, -1, -1]]).astype(np.int32)
    idx_pad = np.concatenate([case["kv_indices"], pad_slots]).astype(np.int32)
    a = orc.verify_attention_ragged(case["q"], case["pool"], case["kv_indices"], case["prefix_lens"], [5],
                                    case["tree_parent"], SCALE)
    b = orc.verify_attention(q_pad, case["pool"], idx_pad, case["prefix_lens"], par_pad[None, :], SCALE)
    np.testing.assert_allclose(a[0], b[0][:5], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(a[1], b[1][:5], rtol=0, atol=1e-13)


def test_ragged_rejects_bad_shapes():
    case = _ragged_case(73, [3, 4], [2, 3])
    with pytest.raises(ValueError):
        orc.verify_attention_ragged(case["q"], case["pool"], case["kv_indices"], case["prefix_lens"], [2, 0],
                                    case["tree_parent"], SCALE)
    with pytest.raises(ValueError):
        orc.verify_attention_ragged(case["q"], case["pool"], case["kv_indices"][:-1], case["prefix_lens"], [2, 3],
                                    case["tree_parent"], SCALE)
