"""GPU parity of the upstream cache write (dsa_cache_write) against the CPU
oracle on the same seeded inputs.  Both sides compute in double precision
and round once to bf16, so every output is compared bit for bit: the whole
latent and indexer caches (rows that must stay untouched included) and the
roped query tensors.  Cases: the 16k chunk's 4096 new tokens (the launch the
benchmark times), eight decode tokens scattered over a 64k-row cache, small
ragged sets with positions -1 and N (rows not written), and calls without
the optional operands."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import dev, host, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

CASES = ["tiny", "glm_small", "glm_decode_8", "glm_16k_chunk"]


def run_gpu(cfg, d, with_index=True, with_q=True):
    import torch
    import sparse_attention_scores_amd as dsa
    kv = dev(d["kv_cache"])
    kI = dev(d["kI_cache"]) if with_index else None
    q = dev(d["q"]) if with_q else None
    qI = dev(d["qI"]) if with_q else None
    pos = torch.from_numpy(d["pos"].astype(np.int32)).cuda()
    dsa.dsa_cache_write(cfg.shape, dev(d["kv_a"]), dev(d["norm_w"]), cfg.eps, pos, cfg.T, cfg.N, kv,
                        dev(d["kI_new"]) if with_index else None, kI, q, qI,
                        d_idx_rope=cfg.d_idx_rope, rope_theta=cfg.theta)
    return (host(kv), None if kI is None else host(kI), None if q is None else host(q),
            None if qI is None else host(qI))


def run_oracle(cfg, d, with_index=True, with_q=True):
    return oracle.cache_write(d["kv_a"], d["norm_w"], cfg.eps, d["pos"], d["kv_cache"],
                              d["kI_new"] if with_index else None, d["kI_cache"] if with_index else None,
                              d["q"] if with_q else None, d["qI"] if with_q else None,
                              shape=cfg.shape, d_idx_rope=cfg.d_idx_rope, theta=cfg.theta)


def same(name, got, want):
    assert got.shape == want.shape, (name, got.shape, want.shape)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, "%s: %d of %d bf16 values differ (first at %d: %#x vs %#x)" % (
        name, bad.size, got.size, bad[0], got.ravel()[bad[0]], want.ravel()[bad[0]])


@pytest.mark.parametrize("name", CASES)
def test_cache_write_matches_oracle(name):
    cfg = W.CACHE_WRITE[name]
    d = W.make_cache_write(cfg)
    say("cache_write", name, "T=%d N=%d" % (cfg.T, cfg.N))
    got = run_gpu(cfg, d)
    want = run_oracle(cfg, d)
    for what, g, w in zip(("kv", "kI", "q", "qI"), got, want):
        same(what, g, w)
    # the write changed what it should: every in-range row, and the rope columns
    good = (d["pos"] >= 0) & (d["pos"] < cfg.N)
    assert not np.array_equal(got[0][d["pos"][good]], d["kv_cache"][d["pos"][good]])


@pytest.mark.parametrize("name", ["tiny", "glm_small"])
def test_cache_write_without_optional_operands(name):
    cfg = W.CACHE_WRITE[name]
    d = W.make_cache_write(cfg)
    say("cache_write (latent only)", name)
    kv, kI, q, qI = run_gpu(cfg, d, with_index=False, with_q=False)
    want = run_oracle(cfg, d, with_index=False, with_q=False)
    assert kI is None and q is None and qI is None
    same("kv", kv, want[0])
