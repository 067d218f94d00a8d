"""dsa_decode_step_noalloc (the decode step over the library's own device
array instead of a caller workspace) against dsa_decode_step, through the C
ABI: the same selections bit for bit and the same outputs within the
attention tolerance, on two calls in a row, the second with a smaller batch
and shorter contexts; a step too large for the array is refused before
anything is enqueued."""
import ctypes

import numpy as np
import pytest

import workloads as W
from tests.gpu_util import ATTN_TOL, dev, host, requires_gpu, row_rel_err, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def _run(cfg, d, noalloc):
    import torch
    import sparse_attention_scores_amd as dsa
    B = len(cfg.ctx)
    out = torch.full((B, cfg.shape.n_heads, cfg.shape.d_latent), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((B, cfg.shape.top_k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    args = (cfg.shape, cfg.ctx, dev(d["q"]), dev(d["qI"]), dev(d["w"]), dev(d["kv"]), dev(d["kI"]), out, idx, cnt)
    if noalloc:
        dsa.dsa_decode_step_noalloc(*args)
    else:
        ws = torch.empty((dsa.dsa_decode_workspace_bytes(cfg.shape, cfg.ctx),), dtype=torch.uint8, device="cuda")
        dsa.dsa_decode_step(*args, ws)
    return host(out), host(idx), host(cnt)


def test_noalloc_matches_workspace_entry_twice():
    big, small = W.DECODE["glm_decode_8"], W.DECODE["glm_decode_small"]
    for cfg in (big, small):          # second call: fewer sequences, shorter contexts
        d = W.make_decode(cfg)
        say("decode-noalloc", cfg.name, cfg.ctx)
        o_ref, i_ref, c_ref = _run(cfg, d, noalloc=False)
        o, i, c = _run(cfg, d, noalloc=True)
        assert np.array_equal(c, c_ref)
        assert np.array_equal(i, i_ref)
        err = row_rel_err(o, o_ref)
        say("decode-noalloc", cfg.name, "max row-relative difference %.3e" % err,
            "bitwise equal" if np.array_equal(o.view(np.uint32), o_ref.view(np.uint32)) else "")
        assert err <= ATTN_TOL, err


def test_noalloc_refuses_oversized_step():
    import sparse_attention_scores_amd as dsa
    ctx = [65536] * 128
    assert dsa.dsa_decode_workspace_bytes(W.GLM, ctx) > dsa.DECODE_STATIC_SCRATCH_BYTES
    arr = (ctypes.c_int64 * len(ctx))(*ctx)
    f = ctypes.c_void_p(0x1000)
    rc = dsa.lib.dsa_decode_step_noalloc(ctypes.byref(dsa.GLM), len(ctx), ctypes.cast(arr, ctypes.c_void_p),
                                         f, f, f, f, f, f, None, None, None)
    assert rc == -3   # DSA_ERR_WORKSPACE, nothing enqueued
