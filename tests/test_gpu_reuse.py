"""Indexer reuse across layers, through the C ABI: the selection one layer's
prefill chunk returns (idx, count) is the selection the next layers attend
with, each over its own queries and latent cache (exo PR #2539: the DSA
indexer is shared across layers).  The chain on the GPU is
dsa_prefill_chunk (layer A) -> dsa_latent_to_f16 + dsa_sparse_mla_attn_f16
and dsa_sparse_mla_attn (layer B, same idx and count, device buffers passed
straight on).  The oracle runs the same chain: its chunk for layer A, then
its attention for layer B over the oracle's own selection.

Bars as for the chunk: selection index-exact, attention <= 2e-3 row-relative.
Layer B's inputs are another seeded draw of the same shapes and positions."""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import ATTN_TOL, dev, host, requires_gpu, row_rel_err, say

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.mark.parametrize("name", ["tiny", "glm_small_cross", "glm_small_first"])
def test_selection_reused_by_next_layer(name):
    import torch
    import sparse_attention_scores_amd as dsa
    cfg = W.PREFILL[name]
    sh = cfg.shape
    da = W.make_prefill(cfg)
    db = W.make_prefill(dataclasses.replace(cfg, seed=cfg.seed + 100))
    say("reuse", name, "L", cfg.L, "q_start", cfg.q_start)
    out_a = torch.empty((cfg.L, sh.n_heads, sh.d_latent), dtype=torch.float32, device="cuda")
    idx = torch.empty((cfg.L, sh.top_k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((cfg.L,), dtype=torch.int32, device="cuda")
    ws = torch.empty((dsa.dsa_prefill_workspace_bytes(sh, cfg.L, cfg.N, cfg.q_start),), dtype=torch.uint8,
                     device="cuda")
    dsa.dsa_prefill_chunk(sh, dev(da["q"]), dev(da["qI"]), dev(da["w"]), dev(da["kv"]), dev(da["kI"]),
                          cfg.L, cfg.N, cfg.q_start, out_a, idx, cnt, ws)
    # layer B: its own queries and cache, layer A's selection as it stands on the device
    q_b, kv_b = dev(db["q"]), dev(db["kv"])
    kv_b16 = torch.empty_like(kv_b)
    dsa.dsa_latent_to_f16(sh, kv_b, cfg.N, kv_b16)
    out_b16 = torch.empty_like(out_a)
    dsa.dsa_sparse_mla_attn_f16(sh, q_b, kv_b16, idx, cnt, cfg.L, cfg.N, out_b16, None)
    out_b = torch.empty_like(out_a)
    dsa.dsa_sparse_mla_attn(sh, q_b, kv_b, idx, cnt, cfg.L, cfg.N, out_b, None)

    ref_idx, ref_cnt, ref_a = oracle.prefill_chunk(da, sh, cfg.q_start)
    assert np.array_equal(host(cnt), ref_cnt)
    assert np.array_equal(host(idx), ref_idx)
    assert row_rel_err(host(out_a), ref_a) <= ATTN_TOL
    ref_b = oracle.sparse_mla_attn(db["q"], db["kv"], ref_idx, ref_cnt, sh.d_latent, sh.softmax_scale)
    for got in (host(out_b16), host(out_b)):
        err = row_rel_err(got, ref_b)
        assert err <= ATTN_TOL, err
    # the layers differ, so the outputs must too (the selection alone is shared)
    assert not np.allclose(host(out_b), host(out_a))
