"""mlaverify_run under HIP graph capture: captured on a non-default stream, replayed
several times with eager work in between, after the device inputs change in place;
every replay must equal the eager result bit for bit.  Capture itself fails if run
synchronises or allocates, so a successful capture also checks that."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, upload, verifier_for
from workloads import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("config", [1, 4])
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
