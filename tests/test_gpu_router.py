"""GPU parity of the router selection (dsa_router_topk) against the CPU
oracle on the same seeded logits and biases.  The expert ids must match bit
for bit (both sides take the decision on the same float32 values: the
sigmoid evaluated in double and rounded once, plus the bias in float
arithmetic; ties to the lower expert).  The weights are formed in double in
selection order on both sides; the GPU rounds them to float, so they must
agree within one float rounding (2^-24 relative).  Cases: the 16k chunk's
4096 tokens (the launch the benchmark times), 8 decode tokens, heavily tied
inputs, probabilities below the weight-sum clamp, and a 64-expert shape."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import dev, host, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.mark.parametrize("name", list(W.ROUTER))
def test_router_matches_oracle(name):
    import torch
    import sparse_attention_scores_amd as dsa
    cfg = W.ROUTER[name]
    d = W.make_router(cfg)
    say("router", name, "T=%d E=%d k=%d" % (cfg.T, cfg.E, cfg.k))
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    dsa.dsa_router_topk(dev(d["logits"]), dev(d["bias"]), cfg.T, cfg.E, cfg.k, cfg.scale, ids, wts)
    gi, gw = host(ids), host(wts)
    oi, ow = oracle.router_topk(d["logits"], d["bias"], cfg.k, cfg.scale)
    bad = np.argwhere(gi != oi)
    assert bad.size == 0, "%d ids differ, first at %s: %d vs %d" % (
        len(bad), bad[0], gi[tuple(bad[0])], oi[tuple(bad[0])])
    err = np.abs(gw.astype(np.float64) - ow) / np.abs(ow)
    assert err.max() <= 2.0 ** -24, float(err.max())
