"""GPU parity of greedy tree acceptance (mlaverify_accept) against its CPU oracle, through the C ABI.

The outputs are integers decided by comparisons of fp32 logits made in fp32 on both sides,
so they must match exactly: accepted length, path, bonus token and error bits.
"""

import numpy as np
import pytest
import torch

import mla_tree_verify_mlaverify_amd as mv
from gpu_util import DEV, i32
from oracle import accept_oracle as acc
from workloads import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run(cfg, max_batch=None):
    b, t = cfg["tree_parent"].shape
    v = mv.Verifier(num_heads=1, max_batch=max_batch or b, max_tree_nodes=t, max_prefix_len=1, pool_slots=1,
                    device=DEV)
    v.read_device_errors()
    lens, path, bonus = v.accept(torch.from_numpy(cfg["logits"]).to(DEV), i32(cfg["draft_tokens"]),
                                 i32(cfg["tree_parent"]))
    torch.cuda.synchronize()
    return lens.cpu().numpy(), path.cpu().numpy(), bonus.cpu().numpy(), v.read_device_errors()


def check(cfg, **kw):
    got = run(cfg, **kw)
    ref = acc.accept(cfg["logits"], cfg["draft_tokens"], cfg["tree_parent"])
    assert np.array_equal(got[0], ref[0]), (got[0], ref[0])
    assert np.array_equal(got[1], ref[1])
    assert np.array_equal(got[2], ref[2])
    assert got[3] == ref[3]
    return got


@pytest.mark.parametrize("seed,b,t,vocab", [
    (0, 1, 1, 1), (1, 1, 8, 16), (2, 4, 33, 1000), (3, 3, 17, 1003), (4, 8, 64, 131072), (5, 2, 64, 50001),
    (6, 16, 5, 7), (7, 1, 64, 16384), (8, 2, 40, 16388), (9, 2, 200, 5000), (10, 1, 256, 1000), (11, 3, 65, 64),
])
def test_accept_matches_oracle(seed, b, t, vocab):
    cfg = synth.accept_config(seed, batch=b, tree_nodes=t, vocab=vocab)
    lens, _, _, _ = check(cfg)
    if vocab > 8:  # the planted paths are found (they may be extended by chance)
        assert all(lens[r] >= len(cfg["planted"][r]) for r in range(b))


def test_special_values():
    cfg = synth.accept_config(11, batch=6, tree_nodes=12, vocab=64, plant=False)
    lg = cfg["logits"]
    lg[0, 0, :] = np.nan                     # a row of NaN: index 0
    lg[1, 0, :] = -np.inf
    lg[1, 0, ::3] = np.nan                   # -inf ranks above NaN
    lg[2, 0, :] = 1.0                        # all equal: lowest index
    lg[3, 0, :] = 0.0
    lg[3, 0, :5] = -0.0                      # -0 ties with +0: lowest index
    lg[4, 0, 7] = np.inf
    lg[4, 0, 9] = np.inf                     # two +inf: the first
    lg[5, 0, :] = -3.0e38
    lg[5, 0, 60] = -2.9e38
    for b in range(6):                       # let row 0's winner be a first-level token
        roots = np.nonzero(cfg["tree_parent"][b] == -1)[0]
        cfg["draft_tokens"][b, roots[0]] = acc.argmax_row(lg[b, 0])
    check(cfg)


def test_bad_tree_accepts_nothing_and_reports():
    cfg = synth.accept_config(12, batch=3, tree_nodes=9, vocab=100)
    cfg["tree_parent"][1, 4] = 6             # a parent after its node
    got = check(cfg)
    assert got[0][1] == 0 and got[3] == mv.DEVERR_BAD_PARENT


def test_batch_below_the_handle_maximum():
    cfg = synth.accept_config(13, batch=2, tree_nodes=16, vocab=300)
    check(cfg, max_batch=8)


def test_repeated_calls_on_one_handle():
    """The workspace is left clean by each call: different trees and sizes in a row agree
    with the oracle every time."""
    v = mv.Verifier(num_heads=1, max_batch=4, max_tree_nodes=40, max_prefix_len=1, pool_slots=1, device=DEV)
    for k, (b, t, vocab) in enumerate([(4, 40, 5000), (1, 3, 9), (4, 40, 5000), (2, 17, 70000), (3, 1, 2)]):
        cfg = synth.accept_config(40 + k, batch=b, tree_nodes=t, vocab=vocab)
        lens, path, bonus = v.accept(torch.from_numpy(cfg["logits"]).to(DEV), i32(cfg["draft_tokens"]),
                                     i32(cfg["tree_parent"]))
        ref = acc.accept(cfg["logits"], cfg["draft_tokens"], cfg["tree_parent"])
        assert np.array_equal(lens.cpu().numpy(), ref[0]) and np.array_equal(path.cpu().numpy(), ref[1])
        assert np.array_equal(bonus.cpu().numpy(), ref[2])
