"""GPU parity: every HIP entry point against the CPU oracle on the same seeded
inputs.  Indexer scores and selections must match bit for bit (integer
indexer data makes every fp32 sum exact); attention must hold a row
relative error of 2e-3 (max over (query, head) of max|o-r| / max|r|).

Small configs are compared on every row.  The full GLM-shape configs run in
the launch configuration the benchmark times: their selections (indices and
counts) are compared with the oracle's on every query row; indexer scores on
one row of every 16-query block (each row over all its keys, so every key
tile is covered); attention on 512 rows spread over the chunk.  Each
attention test prints the error it measured."""
import functools

import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import ATTN_TOL, dev, host, requires_gpu, row_rel_err, say

pytestmark = [pytest.mark.gpu, requires_gpu]

SMALL = ["tiny", "tiny_dense", "tiny_sharp", "glm_small_cross", "glm_small_sparse", "glm_small_first"]
FULL = ["glm_first_4k", "glm_8k", "glm_16k"]


@functools.lru_cache(maxsize=2)
def prefill_inputs(name):
    return W.make_prefill(W.PREFILL[name])


@functools.lru_cache(maxsize=3)
def full_selection(name):
    """The oracle's selection (idx [L, top_k], count [L]) for every query row
    of a chunk: its indexer scores over all keys, then its top-k."""
    cfg = W.PREFILL[name]
    d = prefill_inputs(name)
    S = oracle.indexer_scores(d["qI"], d["kI"], d["w"], cfg.q_start)
    pos = cfg.q_start + np.arange(cfg.L)
    return oracle.topk_select(S, pos, cfg.shape.top_k)


def block_rows(L, block=16, must=()):
    """One row in every block of `block` consecutive queries (its offset in
    the block varies from block to block), plus the rows in `must`."""
    b = np.arange((L + block - 1) // block)
    rows = set(int(x) for x in np.minimum(block * b + (7 * b + 3) % block, L - 1))
    rows.update(int(m) for m in must if 0 <= m < L)
    rows.update([0, L - 1])
    return np.array(sorted(rows), dtype=np.int64)


def lib():
    import sparse_attention_scores_amd as dsa
    return dsa


def run_indexer(cfg, d):
    import torch
    S = torch.empty((cfg.L, cfg.N), dtype=torch.float32, device="cuda")
    lib().dsa_indexer_scores(cfg.shape, dev(d["qI"]), dev(d["kI"]), dev(d["w"]), cfg.L, cfg.N, cfg.q_start, S)
    return S


def run_prefill(cfg, d):
    import torch
    dsa = lib()
    out = torch.empty((cfg.L, cfg.shape.n_heads, cfg.shape.d_latent), dtype=torch.float32, device="cuda")
    idx = torch.empty((cfg.L, cfg.shape.top_k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((cfg.L,), dtype=torch.int32, device="cuda")
    ws = torch.empty((dsa.dsa_prefill_workspace_bytes(cfg.shape, cfg.L, cfg.N, cfg.q_start),),
                     dtype=torch.uint8, device="cuda")
    dsa.dsa_prefill_chunk(cfg.shape, dev(d["q"]), dev(d["qI"]), dev(d["w"]), dev(d["kv"]), dev(d["kI"]),
                          cfg.L, cfg.N, cfg.q_start, out, idx, cnt, ws)
    return host(out), host(idx), host(cnt)


def run_attention(shape, q, kv, idx, cnt, L, N, out, lse, variant):
    """dsa_sparse_mla_attn on a bf16 cache, or dsa_sparse_mla_attn_f16 on the
    fp16-latent copy dsa_latent_to_f16 makes of it (all device tensors)."""
    import torch
    dsa = lib()
    if variant == "bf16":
        dsa.dsa_sparse_mla_attn(shape, q, kv, idx, cnt, L, N, out, lse)
    else:
        kv16 = torch.empty_like(kv)
        dsa.dsa_latent_to_f16(shape, kv, N, kv16)
        dsa.dsa_sparse_mla_attn_f16(shape, q, kv16, idx, cnt, L, N, out, lse)


def check_selection_properties(idx, cnt, pos, top_k):
    """Every row: count = min(p+1, top_k), ascending ids in [0, p], -1 padding."""
    want = np.minimum(pos + 1, top_k)
    assert np.array_equal(cnt, want)
    for r in range(idx.shape[0]):
        c = cnt[r]
        sel = idx[r, :c]
        assert sel[0] >= 0 and sel[-1] <= pos[r], r
        assert np.all(np.diff(sel) > 0), r
        assert np.all(idx[r, c:] == -1), r


# ---------------------------------------------------------------- indexer
@pytest.mark.parametrize("name", SMALL)
def test_indexer_small_bit_exact(name):
    cfg = W.PREFILL[name]
    d = prefill_inputs(name)
    say("indexer", name, cfg.L, cfg.N, cfg.q_start)
    S = host(run_indexer(cfg, d))
    ref = oracle.indexer_scores(d["qI"], d["kI"], d["w"], cfg.q_start)
    assert np.array_equal(S, ref)


@pytest.mark.parametrize("name", FULL)
def test_indexer_full_blocks_bit_exact(name):
    """One row per 16-query block (256+ rows), every key of each row."""
    cfg = W.PREFILL[name]
    d = prefill_inputs(name)
    say("indexer-full", name)
    S = run_indexer(cfg, d)
    rows = block_rows(cfg.L, must=[W.GLM.top_k - cfg.q_start, W.GLM.top_k - cfg.q_start - 1])
    assert rows.size >= 256
    got = host(S[rows.tolist()])
    ref = oracle.indexer_scores(d["qI"], d["kI"], d["w"], cfg.q_start, rows=rows)
    diff = int((got.view(np.uint32) != ref.view(np.uint32)).sum())
    say("indexer-full", name, "rows", rows.size, "differing scores", diff)
    assert diff == 0


# ---------------------------------------------------------------- top-k
@pytest.mark.parametrize("name", SMALL)
def test_topk_small_bit_exact(name):
    import torch
    cfg = W.PREFILL[name]
    d = prefill_inputs(name)
    S = oracle.indexer_scores(d["qI"], d["kI"], d["w"], cfg.q_start)
    pos = cfg.q_start + np.arange(cfg.L)
    ref_idx, ref_cnt = oracle.topk_select(S, pos, cfg.shape.top_k)
    idx = torch.empty((cfg.L, cfg.shape.top_k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((cfg.L,), dtype=torch.int32, device="cuda")
    say("topk", name)
    lib().dsa_topk_select(cfg.shape, dev(S), cfg.L, cfg.N, cfg.q_start, idx, cnt)
    assert np.array_equal(host(cnt), ref_cnt)
    assert np.array_equal(host(idx), ref_idx)


@pytest.mark.parametrize("N,top_k,levels", [(300, 32, 3), (5000, 2048, 5), (16384, 2048, 40),
                                            (16384, 2048, 2), (65536, 2048, 7), (3000, 1, 4),
                                            (2049, 2048, 2), (65537, 2048, 2), (131072, 2048, 7),
                                            (200001, 100, 3), (262144, 2048, 40), (1000, 100, 7),
                                            (2000, 500, 9), (4000, 1000, 50), (8000, 2048, 1000),
                                            (30000, 2048, 40)])
def test_topk_ties_and_sizes(N, top_k, levels):
    """Scores drawn from a few values (many ties at the boundary), negative
    values and -0.0/+0.0 included; every row at a different length."""
    import dataclasses
    import torch
    rng = np.random.default_rng(N + top_k + levels)
    L = 6
    S = (rng.integers(0, levels, size=(L, N)) - levels // 2).astype(np.float32)
    S[S == 0] = np.where(rng.random((S == 0).sum()) < 0.5, -0.0, 0.0).astype(np.float32)
    q_start = N - L
    pos = q_start + np.arange(L)
    ref_idx, ref_cnt = oracle.topk_select(S, pos, top_k)
    shape = dataclasses.replace(W.GLM, top_k=top_k)
    idx = torch.empty((L, top_k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((L,), dtype=torch.int32, device="cuda")
    say("topk-ties", N, top_k, levels)
    lib().dsa_topk_select(shape, dev(S), L, N, q_start, idx, cnt)
    assert np.array_equal(host(cnt), ref_cnt)
    assert np.array_equal(host(idx), ref_idx)


@pytest.mark.parametrize("N,top_k", [(700, 100), (1500, 512), (3500, 2048), (7000, 2048), (12000, 2048),
                                     (30000, 2048), (60000, 2048), (100000, 2048)])
def test_topk_distinct_every_block_shape(N, top_k):
    """Distinct scores (normal, some rows shifted far from zero, one row of
    both signs around a tiny spread) at lengths that reach every block shape
    of the selection: 256 threads with 4 to 32 keys each, 512 x 32,
    1024 x 32, 1024 x 64, and rows taken in pieces."""
    import dataclasses
    import torch
    rng = np.random.default_rng(N + top_k)
    L = 5
    S = rng.standard_normal((L, N)).astype(np.float32)
    S[1] = (S[1] * 0.001 + 1000.0).astype(np.float32)   # narrow range far from zero
    S[2] = (S[2] * 1e-6).astype(np.float32)             # tiny values of both signs
    S[3] = (S[3] * 1e4).astype(np.float32)
    q_start = N - L
    pos = q_start + np.arange(L)
    ref_idx, ref_cnt = oracle.topk_select(S, pos, top_k)
    shape = dataclasses.replace(W.GLM, top_k=top_k)
    idx = torch.empty((L, top_k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((L,), dtype=torch.int32, device="cuda")
    say("topk-distinct", N, top_k)
    lib().dsa_topk_select(shape, dev(S), L, N, q_start, idx, cnt)
    assert np.array_equal(host(cnt), ref_cnt)
    assert np.array_equal(host(idx), ref_idx)


@pytest.mark.parametrize("N", [65600, 150000, 262144])
def test_topk_long_rows_boundary_ties(N):
    """Rows longer than one block's 65536 keys are selected in pieces that
    carry the kept keys forward.  Normal scores with the value ranked near
    top_k planted on keys spread over every piece, so the ties at the
    boundary span pieces and the lower keys must win."""
    import torch
    rng = np.random.default_rng(N)
    L, top_k = 4, 2048
    S = rng.standard_normal((L, N)).astype(np.float32)
    for r in range(L):
        v = np.sort(S[r])[::-1][top_k - 10]
        S[r, rng.choice(N - L, size=60, replace=False)] = v   # 60 keys at the boundary value
    q_start = N - L
    pos = q_start + np.arange(L)
    ref_idx, ref_cnt = oracle.topk_select(S, pos, top_k)
    idx = torch.empty((L, top_k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((L,), dtype=torch.int32, device="cuda")
    say("topk-long", N)
    lib().dsa_topk_select(W.GLM, dev(S), L, N, q_start, idx, cnt)
    assert np.array_equal(host(cnt), ref_cnt)
    assert np.array_equal(host(idx), ref_idx)


@pytest.mark.parametrize("case", ["inf", "wide", "tiny_range", "denormal"])
def test_topk_extreme_values(case):
    """Rows the value-binned levels cannot split (infinities, ranges too wide
    or too narrow for fp32 bins, denormals): the exact fallback must still
    match the brute-force oracle bit for bit."""
    import dataclasses
    import torch
    rng = np.random.default_rng({"inf": 1, "wide": 2, "tiny_range": 3, "denormal": 4}[case])
    L, N, top_k = 5, 12000, 2048
    if case == "inf":
        S = rng.integers(-50, 50, size=(L, N)).astype(np.float32)
        S[:, rng.choice(N, 300, replace=False)] = np.inf
        S[:, rng.choice(N, 300, replace=False)] = -np.inf
    elif case == "wide":
        S = (rng.standard_normal((L, N)) * 10.0 ** rng.integers(-30, 30, size=(L, N))).astype(np.float32)
        S[:, :3] = [3.0e38, -3.0e38, 1.0e-38]
    elif case == "tiny_range":
        base = np.float32(1000.0)
        S = (base + rng.integers(0, 40, size=(L, N)).astype(np.float32) * np.float32(2.0 ** -13)).astype(np.float32)
    else:
        S = (rng.integers(-1000, 1000, size=(L, N)) * np.float32(1e-42)).astype(np.float32)
    q_start = N - L
    pos = q_start + np.arange(L)
    ref_idx, ref_cnt = oracle.topk_select(S, pos, top_k)
    shape = dataclasses.replace(W.GLM, top_k=top_k)
    idx = torch.empty((L, top_k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((L,), dtype=torch.int32, device="cuda")
    say("topk-extreme", case)
    lib().dsa_topk_select(shape, dev(S), L, N, q_start, idx, cnt)
    assert np.array_equal(host(cnt), ref_cnt)
    assert np.array_equal(host(idx), ref_idx)


@pytest.mark.parametrize("case", ["near_zero", "on_edges", "on_edges_scaled"])
def test_topk_bin_edges(case):
    """Keys whose scores sit exactly on the edges of the value bins, and a
    boundary bin around zero (scores of both signs; the selection's last
    level bins a range of a few thousandths across zero, where the floats
    are dense and the bin edges have to be found by a full search): the
    kernel's membership tests must match the bins exactly."""
    import dataclasses
    import torch
    rng = np.random.default_rng({"near_zero": 11, "on_edges": 12, "on_edges_scaled": 13}[case])
    L = 4
    if case == "near_zero":
        N, top_k = 6000, 600
        S = np.concatenate([rng.uniform(-550, -1, (L, 5000)), rng.uniform(-2e-3, 3e-3, (L, 1000))], axis=1)
        S = rng.permuted(S, axis=1).astype(np.float32)
    elif case == "on_edges":   # range [0, 256]: bin edges at the integers
        N, top_k = 12000, 2048
        S = rng.integers(0, 257, size=(L, N)).astype(np.float32)
        S[:, 0], S[:, 1] = 0.0, 256.0
    else:                      # range [-3, 5]: bin edges at multiples of 1/32
        N, top_k = 12000, 2048
        S = (rng.integers(0, 257, size=(L, N)) / 32.0 - 3.0).astype(np.float32)
        S[:, 0], S[:, 1] = -3.0, 5.0
    q_start = N - L
    pos = q_start + np.arange(L)
    ref_idx, ref_cnt = oracle.topk_select(S, pos, top_k)
    shape = dataclasses.replace(W.GLM, top_k=top_k)
    idx = torch.empty((L, top_k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((L,), dtype=torch.int32, device="cuda")
    say("topk-edges", case)
    lib().dsa_topk_select(shape, dev(S), L, N, q_start, idx, cnt)
    assert np.array_equal(host(cnt), ref_cnt)
    assert np.array_equal(host(idx), ref_idx)


@pytest.mark.parametrize("name", FULL)
def test_topk_full_every_row_bit_exact(name):
    """The standalone top-k on the GPU's scores: every row's selection equals
    the oracle's (its own scores and top-k)."""
    import torch
    cfg = W.PREFILL[name]
    d = prefill_inputs(name)
    say("topk-full", name)
    S = run_indexer(cfg, d)
    idx = torch.empty((cfg.L, cfg.shape.top_k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((cfg.L,), dtype=torch.int32, device="cuda")
    lib().dsa_topk_select(cfg.shape, S, cfg.L, cfg.N, cfg.q_start, idx, cnt)
    idx_h, cnt_h = host(idx), host(cnt)
    pos = cfg.q_start + np.arange(cfg.L)
    check_selection_properties(idx_h, cnt_h, pos, cfg.shape.top_k)
    ref_idx, ref_cnt = full_selection(name)
    bad = np.flatnonzero((idx_h != ref_idx).any(axis=1) | (cnt_h != ref_cnt))
    say("topk-full", name, "rows", cfg.L, "differing rows", bad.size, bad[:8].tolist())
    assert bad.size == 0


# ---------------------------------------------------------------- attention
@pytest.mark.parametrize("shape_name", ["TINY", "GLM"])
def test_latent_to_f16_bit_exact(shape_name):
    """Latent columns converted bf16 -> fp16 with round to nearest even
    (numpy's float32 -> float16 is that rounding), rope columns copied; values
    span normal, fp16-subnormal, overflowing and signed-zero cases."""
    import torch
    shape = getattr(W, shape_name)
    rng = np.random.default_rng(7)
    N = 1000
    x = (rng.standard_normal((N, shape.d_qk)) * 10.0 ** rng.integers(-9, 6, size=(N, shape.d_qk))).astype(np.float32)
    x[0, :4] = [0.0, -0.0, 70000.0, -1.0e-30]
    kv = W.to_bf16_bits(x)
    want = kv.copy()
    lat = W.bf16_bits_to_f32(kv[:, :shape.d_latent]).astype(np.float16)
    want[:, :shape.d_latent] = lat.view(np.uint16)
    kv16 = torch.empty((N, shape.d_qk), dtype=torch.int16, device="cuda")
    say("latent-to-f16", shape_name)
    lib().dsa_latent_to_f16(shape, dev(kv), N, kv16)
    assert np.array_equal(host(kv16), want)


@pytest.mark.parametrize("name", SMALL)
def test_attention_f16_small(name):
    """The fp16-latent kernel (the one the prefill chunk runs) on its own."""
    import torch
    cfg = W.PREFILL[name]
    d = prefill_inputs(name)
    ref_idx, ref_cnt, ref_out = oracle.prefill_chunk(d, cfg.shape, cfg.q_start)
    _, ref_lse = oracle.sparse_mla_attn(d["q"], d["kv"], ref_idx, ref_cnt, cfg.shape.d_latent,
                                        cfg.shape.softmax_scale, want_lse=True)
    out = torch.empty((cfg.L, cfg.shape.n_heads, cfg.shape.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((cfg.L, cfg.shape.n_heads), dtype=torch.float32, device="cuda")
    say("attention-f16", name)
    run_attention(cfg.shape, dev(d["q"]), dev(d["kv"]), dev(ref_idx), dev(ref_cnt), cfg.L, cfg.N, out, lse, "f16")
    err = row_rel_err(host(out), ref_out)
    say("attention-f16", name, "max row-relative error %.3e" % err)
    assert err <= ATTN_TOL, err
    assert np.abs(host(lse) - ref_lse).max() < 1e-4


@pytest.mark.parametrize("name", SMALL)
def test_attention_small(name):
    import torch
    cfg = W.PREFILL[name]
    d = prefill_inputs(name)
    ref_idx, ref_cnt, ref_out = oracle.prefill_chunk(d, cfg.shape, cfg.q_start)
    _, ref_lse = oracle.sparse_mla_attn(d["q"], d["kv"], ref_idx, ref_cnt, cfg.shape.d_latent,
                                        cfg.shape.softmax_scale, want_lse=True)
    out = torch.empty((cfg.L, cfg.shape.n_heads, cfg.shape.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((cfg.L, cfg.shape.n_heads), dtype=torch.float32, device="cuda")
    say("attention", name)
    lib().dsa_sparse_mla_attn(cfg.shape, dev(d["q"]), dev(d["kv"]), dev(ref_idx), dev(ref_cnt), cfg.L, cfg.N,
                              out, lse)
    err = row_rel_err(host(out), ref_out)
    say("attention", name, "max row-relative error %.3e" % err)
    assert err <= ATTN_TOL, err
    assert np.abs(host(lse) - ref_lse).max() < 1e-4


@pytest.mark.parametrize("variant", ["bf16", "f16"])
def test_attention_selection_edge_cases(variant):
    """Unordered selections, -1 and out-of-range ids (skipped), counts above
    top_k (clamped), a single key, and a row with no usable key."""
    import torch
    cfg = W.PREFILL["tiny"]
    d = prefill_inputs("tiny")
    rng = np.random.default_rng(3)
    L, N, k = cfg.L, cfg.N, cfg.shape.top_k
    idx = np.full((L, k), -1, np.int32)
    cnt = np.zeros(L, np.int32)
    for i in range(L):
        c = int(rng.integers(1, k + 1))
        idx[i, :c] = rng.choice(N, size=c, replace=False)
        cnt[i] = c
    idx[1, 3] = N + 5          # out of range: skipped
    idx[2, 0] = -7             # negative: skipped
    cnt[3] = k + 100           # clamped to top_k (padding -1 entries are skipped)
    cnt[4] = 1
    idx[5, :] = -1             # no usable key
    cnt[5] = 4
    ref_out, ref_lse = oracle.sparse_mla_attn(d["q"], d["kv"], idx, np.minimum(cnt, k), cfg.shape.d_latent,
                                              cfg.shape.softmax_scale, want_lse=True)
    out = torch.empty((L, cfg.shape.n_heads, cfg.shape.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((L, cfg.shape.n_heads), dtype=torch.float32, device="cuda")
    say("attention-edge", variant)
    run_attention(cfg.shape, dev(d["q"]), dev(d["kv"]), dev(idx), dev(cnt), L, N, out, lse, variant)
    o, s = host(out), host(lse)
    assert np.all(o[5] == 0.0) and np.all(s[5] == -np.inf)
    keep = np.arange(L) != 5
    assert row_rel_err(o[keep], ref_out[keep]) <= ATTN_TOL
    assert np.abs(s[keep] - ref_lse[keep]).max() < 1e-4
    # the order of a selection does not matter
    idx2 = idx.copy()
    for i in range(L):
        idx2[i, : min(cnt[i], k)] = rng.permutation(idx[i, : min(cnt[i], k)])
    out2 = torch.empty_like(out)
    run_attention(cfg.shape, dev(d["q"]), dev(d["kv"]), dev(idx2), dev(cnt), L, N, out2, None, variant)
    assert row_rel_err(host(out2)[keep], ref_out[keep]) <= ATTN_TOL


# ---------------------------------------------------------------- prefill chunk
@pytest.mark.parametrize("name", SMALL)
def test_prefill_chunk_small(name):
    cfg = W.PREFILL[name]
    d = prefill_inputs(name)
    say("prefill", name)
    out, idx, cnt = run_prefill(cfg, d)
    ref_idx, ref_cnt, ref_out = oracle.prefill_chunk(d, cfg.shape, cfg.q_start)
    assert np.array_equal(cnt, ref_cnt)
    assert np.array_equal(idx, ref_idx)
    err = row_rel_err(out, ref_out)
    say("prefill", name, "max row-relative error %.3e" % err)
    assert err <= ATTN_TOL, err


@pytest.mark.parametrize("name", FULL)
def test_prefill_chunk_full(name):
    """dsa_prefill_chunk as the benchmark runs it: the selection of every row
    equals the oracle's; attention on 512 rows spread over the chunk (the
    top_k boundary rows included) within the tolerance."""
    cfg = W.PREFILL[name]
    d = prefill_inputs(name)
    say("prefill-full", name)
    out, idx, cnt = run_prefill(cfg, d)
    pos = cfg.q_start + np.arange(cfg.L)
    check_selection_properties(idx, cnt, pos, cfg.shape.top_k)
    assert np.all(np.isfinite(out))
    ref_idx, ref_cnt = full_selection(name)
    bad = np.flatnonzero((idx != ref_idx).any(axis=1) | (cnt != ref_cnt))
    say("prefill-full", name, "differing selection rows", bad.size, bad[:8].tolist())
    assert bad.size == 0
    rows = W.sample_rows(cfg.L, 512, seed=7, must=[W.GLM.top_k - cfg.q_start, W.GLM.top_k - cfg.q_start - 1])
    ref_out = oracle.sparse_mla_attn(d["q"], d["kv"], ref_idx, ref_cnt, cfg.shape.d_latent,
                                     cfg.shape.softmax_scale, rows=rows)
    err = row_rel_err(out[rows], ref_out)
    say("prefill-full", name, "attention rows", rows.size, "max row-relative error %.3e" % err)
    assert err <= ATTN_TOL, err


def test_prefill_chunk_fp16_range():
    """The fp16 contract of the hot path: the chunk's attention runs with the
    latent score part and the value product on fp16 operands (the rope part
    stays bf16).  Latent and query values here span fp16's subnormal range
    (most query values and a third of the latent values lie below 2**-14)
    up to magnitudes of 2**15; the chunk must still match the oracle, which
    reads the same bf16 inputs in double precision, within the tolerance."""
    cfg = W.PREFILL["glm_small_cross"]
    d = W.make_prefill_fp16_range(cfg)
    kv = W.bf16_bits_to_f32(d["kv"][:, :cfg.shape.d_latent])
    q = W.bf16_bits_to_f32(d["q"][..., :cfg.shape.d_latent])
    assert np.abs(kv).max() == 2.0 ** 15
    assert (np.abs(kv) < 2.0 ** -14).mean() > 0.25 and (np.abs(q) < 2.0 ** -14).mean() > 0.5
    say("prefill-fp16-range", cfg.L, cfg.N, cfg.q_start)
    out, idx, cnt = run_prefill(cfg, d)
    ref_idx, ref_cnt, ref_out = oracle.prefill_chunk(d, cfg.shape, cfg.q_start)
    assert np.array_equal(cnt, ref_cnt)
    assert np.array_equal(idx, ref_idx)
    err = row_rel_err(out, ref_out)
    say("prefill-fp16-range", "max row-relative error %.3e" % err)
    assert err <= ATTN_TOL, err


def test_prefill_chunk_deterministic():
    cfg = W.PREFILL["glm_small_cross"]
    d = prefill_inputs("glm_small_cross")
    a = run_prefill(cfg, d)
    b = run_prefill(cfg, d)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("L,q_start", [(1, 0), (1, 5000), (3, 2046), (129, 1919), (3, 99997)])
def test_prefill_chunk_edges(L, q_start):
    """One query at position 0 (a single key), one deep query, a chunk that
    straddles the top_k boundary by one, and a ragged 129-query chunk."""
    import dataclasses
    cfg = dataclasses.replace(W.PREFILL["glm_small_cross"], L=L, q_start=q_start, seed=40 + L)
    d = W.make_prefill(cfg)
    say("prefill-edge", L, q_start)
    out, idx, cnt = run_prefill(cfg, d)
    ref_idx, ref_cnt, ref_out = oracle.prefill_chunk(d, cfg.shape, cfg.q_start)
    assert np.array_equal(cnt, ref_cnt)
    assert np.array_equal(idx, ref_idx)
    err = row_rel_err(out, ref_out)
    say("prefill-edge", L, q_start, "max row-relative error %.3e" % err)
    assert err <= ATTN_TOL, err


# ---------------------------------------------------------------- decode
def run_decode(cfg, d):
    import torch
    dsa = lib()
    B = len(cfg.ctx)
    out = torch.empty((B, cfg.shape.n_heads, cfg.shape.d_latent), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, cfg.shape.top_k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    ws = torch.empty((dsa.dsa_decode_workspace_bytes(cfg.shape, cfg.ctx),), dtype=torch.uint8, device="cuda")
    dsa.dsa_decode_step(cfg.shape, cfg.ctx, dev(d["q"]), dev(d["qI"]), dev(d["w"]), dev(d["kv"]), dev(d["kI"]),
                        out, idx, cnt, ws)
    return host(out), host(idx), host(cnt)


@pytest.mark.parametrize("name", ["tiny_decode", "glm_decode_small", "glm_decode_8"])
def test_decode_step(name):
    cfg = W.DECODE[name]
    d = W.make_decode(cfg)
    say("decode", name, cfg.ctx)
    out, idx, cnt = run_decode(cfg, d)
    ref_idx, ref_cnt, ref_out = oracle.decode_step(d, cfg.shape)
    assert np.array_equal(cnt, ref_cnt)
    assert np.array_equal(idx, ref_idx)
    err = row_rel_err(out, ref_out)
    say("decode", name, "max row-relative error %.3e" % err)
    assert err <= ATTN_TOL, err


@pytest.mark.parametrize("name,B", [("tiny", 300), ("glm", 131)])
def test_decode_step_large_batch(name, B):
    """Batches of more than 128 sequences run as groups of 128 that share
    the workspace; every group's operands start at its first sequence.
    Ragged contexts of 1 to 3000 keys (some below top_k, some above)."""
    rng = np.random.default_rng(B)
    shape = W.TINY if name == "tiny" else W.GLM
    ctx = tuple(int(c) for c in rng.integers(1, 3000 if name == "glm" else 700, size=B))
    cfg = W.Decode("batch_%s_%d" % (name, B), shape, ctx, 50 + B, 8 if name == "glm" else 4, 0.05, 0.05)
    d = W.make_decode(cfg)
    say("decode-batch", name, B)
    out, idx, cnt = run_decode(cfg, d)
    ref_idx, ref_cnt, ref_out = oracle.decode_step(d, cfg.shape)
    assert np.array_equal(cnt, ref_cnt)
    assert np.array_equal(idx, ref_idx)
    err = row_rel_err(out, ref_out)
    say("decode-batch", name, B, "max row-relative error %.3e" % err)
    assert err <= ATTN_TOL, err


@pytest.mark.parametrize("case", ["all_ties", "one_segment", "ties_in_bin", "wide_bin", "long", "all_ties_long"])
def test_decode_segmented_topk(case):
    """Decode selection over sequences longer than one segment block (8192
    keys): ties spanning every segment (all scores equal: the first top_k
    keys win), a selection held entirely by one segment (the others' keys
    must all lose; its top_k equal scores fill one bin), and scores from
    1999 values repeated across the sequence, so the bin holding the top_k-th
    key has a few dozen keys with ties inside it, ranked by the final block
    (lower key first); 251 repeated values, whose boundary bins hold 35 to
    260 equal keys (ranked by several waves past 64).  Contexts past 65536
    keys: normal scores over 32
    segments (the histogram counts summed eight segments at a time), and all
    ties, where the final block selects the whole sequence in pieces."""
    ctx = {"ties_in_bin": (65536, 40000, 16385, 8193, 18000), "wide_bin": (65536, 30000, 9000),
           "long": (262144, 70001, 131072),
           "all_ties_long": (262144, 70000)}.get(case, (40000, 16385, 18000))
    cfg = W.Decode("seg_" + case, W.GLM, ctx, 31, 8, 0.05, 0.05)
    d = W.make_decode(cfg)
    top_k = cfg.shape.top_k
    want0 = None
    if case in ("all_ties", "all_ties_long"):
        d["qI"][:] = 0
        want0 = np.arange(top_k)
    elif case == "long":
        pass
    elif case in ("ties_in_bin", "wide_bin"):
        d["qI"][:] = W.to_bf16_bits(np.float32(1.0))   # every q.k is the sum of k
        rows = np.arange(d["kI"].shape[0])
        period = 1999 if case == "ties_in_bin" else 251   # 251 values: boundary bins of 35-260 equal keys
        vals = W.to_bf16_bits(((rows % period) / 128.0).astype(np.float32))
        d["kI"][:] = vals[:, None]
    else:
        one, eight = W.to_bf16_bits(np.float32(1.0)), W.to_bf16_bits(np.float32(8.0))
        d["qI"][0] = one                  # sequence 0: every q.k is the sum of k
        lo = 17000                        # keys 17000..19047 sit in the second segment
        d["kI"][lo:lo + top_k] = eight    # the only keys reaching 128 * 8 per head
        want0 = np.arange(lo, lo + top_k)
    say("decode-seg", case, cfg.ctx)
    out, idx, cnt = run_decode(cfg, d)
    ref_idx, ref_cnt, ref_out = oracle.decode_step(d, cfg.shape)
    if want0 is not None:
        assert np.array_equal(ref_idx[0], want0)
    assert np.array_equal(cnt, ref_cnt)
    assert np.array_equal(idx, ref_idx)
    assert row_rel_err(out, ref_out) <= ATTN_TOL
