"""The decode step and the prefill chunk captured into HIP graphs
(torch.cuda.graph over the binding's current stream): each replay must
equal the eager call bit for bit.  Neither has a memset, copy or
allocation, so the graphs hold only kernels.  Replays are interleaved with eager work on other inputs and
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


def test_prefill_chunk_graph_replays_match_eager():
    """The prefill chunk (indexer, top-k, latent -> fp16, attention over one
    workspace) captured into a graph: every replay equals the eager chunk bit
    for bit (output, selection and counts), with eager chunks on other inputs
    between the replays.  glm_small_cross: 77 queries at 2011..2087, across
    the top_k boundary."""
    import torch
    import sparse_attention_scores_amd as dsa
    cfg = W.PREFILL["glm_small_cross"]
    sh = cfg.shape
    d1 = W.make_prefill(cfg)
    t = {k: dev(d1[k]) for k in ("q", "qI", "w", "kv", "kI")}
    out = torch.empty((cfg.L, sh.n_heads, sh.d_latent), dtype=torch.float32, device="cuda")
    idx = torch.empty((cfg.L, sh.top_k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((cfg.L,), dtype=torch.int32, device="cuda")
    ws = torch.empty((dsa.dsa_prefill_workspace_bytes(sh, cfg.L, cfg.N, cfg.q_start),), dtype=torch.uint8,
                     device="cuda")
    run = lambda tt, o, i, c, w: dsa.dsa_prefill_chunk(sh, tt["q"], tt["qI"], tt["w"], tt["kv"], tt["kI"], cfg.L,
                                                       cfg.N, cfg.q_start, o, i, c, w)
    say("prefill graph", cfg.name, "eager reference")
    run(t, out, idx, cnt, ws)
    ref = (host(out).copy(), host(idx).copy(), host(cnt).copy())
    other = {k: v.clone() for k, v in t.items()}
    other["qI"] = dev(np.ascontiguousarray(np.roll(d1["qI"], 1, axis=0)))
    out2, idx2, cnt2, ws2 = torch.empty_like(out), torch.empty_like(idx), torch.empty_like(cnt), torch.empty_like(ws)
    say("prefill graph", cfg.name, "capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(t, out, idx, cnt, ws)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(t, out, idx, cnt, ws)
    torch.cuda.synchronize()
    for rep in range(4):
        say("prefill graph", cfg.name, "replay", rep)
        out.fill_(float("nan"))
        idx.fill_(-7)
        cnt.fill_(-7)
        run(other, out2, idx2, cnt2, ws2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), ref[0]), rep
        assert np.array_equal(host(idx), ref[1]) and np.array_equal(host(cnt), ref[2]), rep
        run(other, out2, idx2, cnt2, ws2)
    del g
