"""GPU parity of the dense masked path (dsa_selection_mask,
dsa_dense_masked_attn, dsa_values_to_f16 + dsa_dense_masked_attn_f16) against the CPU oracle on the same seeded inputs and
the same selection (the oracle's top-k of seeded indexer scores).

- selection mask: integer work, bit-exact over every row;
- value conversion: bit-exact against numpy's round-to-nearest-even
  float32 -> float16 of the decoded bf16 values, laid out in the vt form
  (feature-major, keys in the tile order, zero padding);
- attention: max over (query, head) rows of max|o - r| / max|r| <= 2e-3.
  The GPU sums bf16 products in fp32, rounds the probabilities to fp16
  (relative 2^-11) and converts the values to fp16 (exact here); the oracle
  is fp64 throughout.  The rounding of the probabilities dominates: about
  2^-11 / sqrt(3) of the row's scale, well inside the bound.
Cases: 160 GLM-width queries over 700 keys (ragged query block and key
tile), two tiny-width chunks (several query blocks and tiles, a first chunk
whose early queries take every earlier key, a row with an empty selection),
the 8k-key chunk the benchmark times (4096 queries, every head; the oracle
runs on a seeded sample of rows), the first 4096-query chunk at GLM widths,
and the widest selection mask the entry takes."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import ATTN_TOL, dev, host, requires_gpu, row_rel_err, say, vt_layout

pytestmark = [pytest.mark.gpu, requires_gpu]


def select(cfg, d, empty_rows=()):
    pos = cfg.q_start + np.arange(cfg.L)
    S = d["S"].copy()
    S[np.arange(cfg.N)[None, :] > pos[:, None]] = -np.inf
    idx, cnt = oracle.topk_select(S, pos, cfg.top_k)
    for r in empty_rows:
        cnt[r] = 0
    return idx, cnt


def run(cfg, empty_rows=(), rows=None):
    import torch
    import sparse_attention_scores_amd as dsa
    d = W.make_dense(cfg)
    idx, cnt = select(cfg, d, empty_rows)
    Wm = dsa.mask_words(cfg.N)
    say("dense", cfg.name, "L", cfg.L, "N", cfg.N, "q_start", cfg.q_start, "H", cfg.H)
    mask = torch.empty((cfg.L, Wm), dtype=torch.int32, device="cuda")
    dsa.dsa_selection_mask(dev(idx), dev(cnt), cfg.L, cfg.top_k, cfg.N, cfg.q_start, mask)
    mask_h = host(mask).view(np.uint32)
    mask_ref = oracle.selection_mask(idx, cnt, cfg.N, cfg.q_start, W=Wm)
    assert np.array_equal(mask_h, mask_ref)
    out = torch.empty((cfg.L, cfg.H, cfg.Dv), dtype=torch.float32, device="cuda")
    dsa.dsa_dense_masked_attn(dev(d["q"]), dev(d["kvb"]), dev(d["kv"]), cfg.Dl + cfg.Dr, cfg.Dl, mask,
                              cfg.L, cfg.N, cfg.q_start, cfg.H, cfg.Dn, cfg.Dr, cfg.Dv, 1.0 / 16, out)
    got = host(out)
    assert np.isfinite(got).all()
    rows = np.arange(cfg.L) if rows is None else rows
    ref = oracle.dense_masked_attn(d["q"], d["kvb"], d["kv"], mask_ref, cfg.Dn, cfg.Dr, cfg.Dv, cfg.Dl,
                                   1.0 / 16, rows=rows)
    err = row_rel_err(got[rows], ref)
    assert err <= ATTN_TOL, err
    for r in empty_rows:
        assert not got[r].any()
    # the fp16-value entry on the same inputs: values converted to the vt form first
    Np = dsa.vt_keys(cfg.N)
    kvb_d = dev(d["kvb"])
    vt = torch.full((cfg.H, cfg.Dv, Np), -1, dtype=torch.int16, device="cuda")   # padding must be written
    dsa.dsa_values_to_f16(kvb_d, cfg.N, cfg.H, cfg.Dn, cfg.Dv, vt)
    want = vt_layout(W.bf16_bits_to_f32(d["kvb"][..., cfg.Dn:]).astype(np.float16).view(np.uint16), Np)
    assert np.array_equal(host(vt), want)
    out16 = torch.empty_like(out)
    dsa.dsa_dense_masked_attn_f16(dev(d["q"]), kvb_d, vt, dev(d["kv"]), cfg.Dl + cfg.Dr, cfg.Dl, mask,
                                  cfg.L, cfg.N, cfg.q_start, cfg.H, cfg.Dn, cfg.Dr, cfg.Dv, 1.0 / 16, out16)
    got16 = host(out16)
    err16 = row_rel_err(got16[rows], ref)
    assert err16 <= ATTN_TOL, err16
    for r in empty_rows:
        assert not got16[r].any()
    return got


def test_dense_tiny():
    run(W.DENSE["tiny"], empty_rows=(3, 199))


def test_dense_tiny_first_chunk():
    run(W.DENSE["tiny_first"])


def test_dense_glm_small():
    run(W.DENSE["glm_small"], empty_rows=(7,))


def test_dense_glm_8k_chunk_sampled():
    cfg = W.DENSE["glm_8k_chunk"]
    run(cfg, rows=W.sample_rows(cfg.L, 12, seed=9, must=[0, 127, 128, cfg.L - 1]))


def test_dense_rejects_bad_arguments():
    import torch
    import sparse_attention_scores_amd as dsa
    cfg = W.DENSE["tiny"]
    q = torch.zeros((cfg.L, cfg.H, 128), dtype=torch.int16, device="cuda")
    kvb = torch.zeros((cfg.N, cfg.H, 128), dtype=torch.int16, device="cuda")
    kv = torch.zeros((cfg.N, 128), dtype=torch.int16, device="cuda")
    mask = torch.zeros((cfg.L, dsa.mask_words(cfg.N)), dtype=torch.int32, device="cuda")
    out = torch.empty((cfg.L, cfg.H, 64), dtype=torch.float32, device="cuda")
    say("dense argument checks")
    with pytest.raises(dsa.DsaError):   # unsupported widths
        dsa.dsa_dense_masked_attn(q, kvb, kv, 128, 64, mask, cfg.L, cfg.N, 0, cfg.H, 48, 16, 64, 0.0625, out)
    with pytest.raises(dsa.DsaError):   # mask rows too short for N
        dsa.dsa_dense_masked_attn(q, kvb, kv, 128, 64, mask[:, :2].contiguous(), cfg.L, cfg.N, 0, cfg.H, 64, 64, 64, 0.0625, out)
    with pytest.raises(dsa.DsaError):   # rope key past the cache row
        dsa.dsa_dense_masked_attn(q, kvb, kv, 128, 72, mask, cfg.L, cfg.N, 0, cfg.H, 64, 64, 64, 0.0625, out)


def test_dense_glm_first_chunk_sampled():
    """The first 4096-query chunk at GLM widths: queries 0..2047 take every
    earlier key (the causal regime the pages route to a causal kernel), the
    rest a real top-2048 selection."""
    cfg = W.DENSE["glm_4k_first"]
    run(cfg, rows=W.sample_rows(cfg.L, 12, seed=10, must=[0, 1, 2046, 2047, 2048, cfg.L - 1]))


def test_selection_mask_widest_rows():
    """The widest mask the entry takes (16384 words: 524288 keys) is written
    bit-exactly, padding and out-of-range ids included; one word wider is
    refused."""
    import torch
    import sparse_attention_scores_amd as dsa
    L, top_k, N = 6, 2048, 524288
    rng = np.random.default_rng(12)
    q_start = N - L
    idx = np.sort(rng.choice(N, size=(L, top_k), replace=True), axis=1).astype(np.int32)
    idx[:, :3] = [-1, N, N + 7]          # ignored entries
    idx[0, -1] = q_start + 5             # after query 0's position: not causal for it
    cnt = np.array([top_k, top_k - 1, 0, 17, top_k, 1000], np.int32)
    say("selection mask widest", N)
    mask = torch.empty((L, dsa.mask_words(N)), dtype=torch.int32, device="cuda")
    dsa.dsa_selection_mask(dev(idx), dev(cnt), L, top_k, N, q_start, mask)
    want = oracle.selection_mask(idx, cnt, N, q_start)
    assert np.array_equal(host(mask).view(np.uint32), want)
    wide = torch.empty((L, dsa.mask_words(N) + 2), dtype=torch.int32, device="cuda")
    with pytest.raises(dsa.DsaError):
        dsa.dsa_selection_mask(dev(idx), dev(cnt), L, top_k, N + 64, q_start, wide)


def test_dense_single_query():
    """One query (a block of one row: 127 query slots and 7 of 8 waves idle)
    at the end of a ragged key range, and one at position 0 (a single key)."""
    import dataclasses
    for q_start, N in ((299, 300), (0, 1)):
        cfg = dataclasses.replace(W.DENSE["tiny"], name="tiny_one_%d" % q_start, L=1, N=N, q_start=q_start)
        run(cfg)
