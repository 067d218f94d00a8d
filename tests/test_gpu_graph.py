"""The decode step captured into a HIP graph (torch.cuda.graph over the
binding's current stream): each replay must equal the eager step bit for
bit.  The step has no memset, copy or allocation, so the graph holds only
its kernels.  Replays are interleaved with eager work on other inputs and
with synchronisations, and every replay is checked, so a node that only
works on its first replay would show."""
import numpy as np
import pytest

import workloads as W
from tests.gpu_util import dev, host, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def test_decode_step_graph_replays_match_eager():
    import torch
    import sparse_attention_scores_amd as dsa
    dc = W.DECODE["glm_decode_small"]
    sh = dc.shape
    B = len(dc.ctx)
    d1 = W.make_decode(dc)
    t = {k: dev(d1[k]) for k in ("q", "qI", "w", "kv", "kI")}
    out = torch.empty((B, sh.n_heads, sh.d_latent), dtype=torch.float32, device="cuda")
    ws = torch.empty((dsa.dsa_decode_workspace_bytes(sh, dc.ctx),), dtype=torch.uint8, device="cuda")
    step = lambda: dsa.dsa_decode_step(sh, dc.ctx, t["q"], t["qI"], t["w"], t["kv"], t["kI"], out, None, None, ws)
    say("decode graph", dc.name, "eager reference")
    step()
    ref = host(out).copy()
    # eager work on other inputs between replays
    other = {k: v.clone() for k, v in t.items()}
    other["q"] = dev(np.ascontiguousarray(np.roll(d1["q"], 1, axis=0)))
    out2 = torch.empty_like(out)
    ws2 = torch.empty_like(ws)
    eager_other = lambda: dsa.dsa_decode_step(sh, dc.ctx, other["q"], other["qI"], other["w"], other["kv"],
                                              other["kI"], out2, None, None, ws2)
    say("decode graph", dc.name, "capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        say("decode graph", dc.name, "replay", rep)
        out.fill_(float("nan"))
        eager_other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), ref), rep
        eager_other()
    del g
