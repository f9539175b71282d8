"""mlaverify_run (on every gather path), mlaverify_run_static, mlaverify_run_ragged on paged
prefixes, mlaverify_relocate and mlaverify_accept under HIP graph capture: captured
on a non-default stream, replayed several times with eager work in between, and after the
device inputs change in place; every replay must equal the eager result bit for bit.
Capture itself fails if a call synchronises or allocates, so a successful capture also
checks that."""

import numpy as np
import pytest
import torch

import mla_tree_verify_mlaverify_amd as mv
from gpu_util import DEV, bf16, i32, upload, verifier_for
from test_gpu_ragged import paged_ragged_case
from workloads import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


# 4k (LDS-DMA gathers), the batch of 8, and the 185k shapes of 64 rows (helper waves) and
# 128 rows (register-staged gathers)
@pytest.mark.parametrize("config", [1, 4, 5, 6])
def test_graph_replay_matches_eager(config):
    cfg = synth.make_config(config)
    d = upload(cfg)
    v = verifier_for(cfg)
    b, t, h = cfg["batch"], cfg["tree_nodes"], cfg["heads"]
    out = torch.empty((b * t, h, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((b * t, h), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        v.run(d["q"], d["pool"], d["kv_indices"], d["prefix_lens"], d["tree_parent"], out=out, lse=lse)
    torch.cuda.synchronize()
    eager_out, eager_lse = out.clone(), lse.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        v.run(d["q"], d["pool"], d["kv_indices"], d["prefix_lens"], d["tree_parent"], out=out, lse=lse)
    torch.cuda.synchronize()

    for rep in range(3):
        out.fill_(0)
        lse.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out), rep
        assert torch.equal(lse, eager_lse), rep
        # eager work between replays on the same handle and buffers
        v.run(d["q"], d["pool"], d["kv_indices"], d["prefix_lens"], d["tree_parent"], out=out, lse=lse)
        torch.cuda.synchronize()

    # new device inputs in place (q and the tree), same shapes: replay must follow them
    rng = np.random.default_rng(5)
    q2 = synth.f32_to_bf16_bits(rng.standard_normal(cfg["q"].shape, dtype=np.float32) * np.float32(0.5))
    par2 = np.stack([synth.chain_tree(t) for _ in range(b)]).astype(np.int32)
    d["q"].copy_(torch.from_numpy(q2.view(np.int16)).view(torch.bfloat16).to(DEV))
    d["tree_parent"].copy_(torch.from_numpy(par2).to(DEV))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    got_out, got_lse = out.clone(), lse.clone()
    v.run(d["q"], d["pool"], d["kv_indices"], d["prefix_lens"], d["tree_parent"], out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(got_out, out) and torch.equal(got_lse, lse)
    assert not torch.equal(got_out, eager_out)


def test_graph_replay_relocation():
    # relocation under capture: each replay starts from the original pool and indices and
    # must leave exactly the eager result (pool bytes and rewritten indices)
    from gpu_util import i32

    cfg = synth.defrag_config(5, batch=3, prefix=[700, 64, 1500], tree_nodes=12, heads=8, slots=8192)
    d = upload(cfg)
    v = verifier_for(cfg)
    t = cfg["tree_nodes"]
    dst = i32(cfg["dst_start"])
    pool0, idx0 = d["pool"].clone(), d["kv_indices"].clone()
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        v.relocate(d["pool"], d["kv_indices"], d["prefix_lens"], dst, t, stream=s)
    torch.cuda.synchronize()
    assert v.read_device_errors() == 0
    eager_pool, eager_idx = d["pool"].clone(), d["kv_indices"].clone()
    assert not torch.equal(eager_idx, idx0)  # something moved
    d["pool"].copy_(pool0)
    d["kv_indices"].copy_(idx0)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        v.relocate(d["pool"], d["kv_indices"], d["prefix_lens"], dst, t, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        d["pool"].copy_(pool0)
        d["kv_indices"].copy_(idx0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d["pool"].view(torch.int16), eager_pool.view(torch.int16)), rep
        assert torch.equal(d["kv_indices"], eager_idx), rep
        # a replay over an already relocated batch moves nothing more
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d["kv_indices"], eager_idx), rep
    assert v.read_device_errors() == 0


def test_graph_replay_acceptance():
    # acceptance under capture: replays equal the eager result, with eager calls on the same
    # handle in between (the walk leaves its workspace keys at zero), and follow new logits
    from gpu_util import i32

    cfg = synth.accept_config(4, batch=8, tree_nodes=64, vocab=131072)
    b, t = cfg["tree_parent"].shape
    v = mv_verifier_for_accept(b, t)
    logits = torch.from_numpy(cfg["logits"]).to(DEV)
    dt, par = i32(cfg["draft_tokens"]), i32(cfg["tree_parent"])
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ref = [x.clone() for x in v.accept(logits, dt, par, stream=s)]
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        outs = v.accept(logits, dt, par, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), rep
        v.accept(logits, dt, par)  # eager work between replays
        torch.cuda.synchronize()

    # new logits in place: the replay must follow them
    logits.copy_(torch.flip(logits, dims=[2]))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    got = [o.clone() for o in outs]
    eager = v.accept(logits, dt, par)
    torch.cuda.synchronize()
    for o, r in zip(got, eager):
        assert torch.equal(o, r)
    assert v.read_device_errors() == 0


def mv_verifier_for_accept(b, t):
    import mla_tree_verify_mlaverify_amd as mv

    return mv.Verifier(num_heads=1, max_batch=b, max_tree_nodes=t, max_prefix_len=1, pool_slots=1, device=DEV)


def _replay_three_times(g, outs, eager, between):
    for rep in range(3):
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), rep
        between()
        torch.cuda.synchronize()


def test_graph_replay_static_entry():
    # the allocation-free entry point captured (its device lookup done by an eager call first)
    cfg = synth.make_config(1)
    d = upload(cfg)
    b, t, h = cfg["batch"], cfg["tree_nodes"], cfg["heads"]
    lc = mv.make_config(h, b, t, int(cfg["prefix_lens"].max()), cfg["slots"], cfg["row_stride"], cfg["sm_scale"])
    out = torch.empty((b * t, h, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((b * t, h), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mv.run_static(lc, d["q"], d["pool"], d["kv_indices"], d["prefix_lens"], d["tree_parent"], out, lse)
    torch.cuda.synchronize()
    eager = (out.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mv.run_static(lc, d["q"], d["pool"], d["kv_indices"], d["prefix_lens"], d["tree_parent"], out, lse)
    torch.cuda.synchronize()
    v = verifier_for(cfg)
    o2 = torch.empty_like(out)
    l2 = torch.empty_like(lse)
    # eager calls of both entry points between the replays
    _replay_three_times(g, (out, lse), eager, lambda: (
        v.run(d["q"], d["pool"], d["kv_indices"], d["prefix_lens"], d["tree_parent"], out=o2, lse=l2),
        mv.run_static(lc, d["q"], d["pool"], d["kv_indices"], d["prefix_lens"], d["tree_parent"], o2, l2)))
    assert torch.equal(o2, eager[0]) and torch.equal(l2, eager[1])


def test_graph_replay_ragged_paged():
    paged, _ = paged_ragged_case(93, [700, 0, 2100, 33], [5, 1, 40, 64], 8, 16384, 16)
    max_t = int(paged["tree_lens"].max())
    v = mv.Verifier(num_heads=8, max_batch=4, max_tree_nodes=max_t, max_prefix_len=2100, pool_slots=16384,
                    sm_scale=paged["sm_scale"], page_size=16, device=DEV)
    q, pool, idx = bf16(paged["q"]), bf16(paged["pool"]), i32(paged["kv_indices"])
    pl, tl, par = i32(paged["prefix_lens"]), i32(paged["tree_lens"]), i32(paged["tree_parent"])
    rows = paged["q"].shape[0]
    out = torch.empty((rows, 8, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((rows, 8), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        v.run_ragged(q, pool, idx, pl, tl, par, max_t, out=out, lse=lse)
    torch.cuda.synchronize()
    eager = (out.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        v.run_ragged(q, pool, idx, pl, tl, par, max_t, out=out, lse=lse)
    torch.cuda.synchronize()
    o2, l2 = torch.empty_like(out), torch.empty_like(lse)
    _replay_three_times(g, (out, lse), eager, lambda: v.run_ragged(q, pool, idx, pl, tl, par, max_t, out=o2, lse=l2))
    assert v.read_device_errors() == 0
