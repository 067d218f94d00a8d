"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a value that does not come from the oracle itself: a hand-worked example
(tests/golden/), an exact rational brute force on tiny inputs, a closed
form, an invariant, or a special case that reduces to a library routine
(torch's scaled_dot_product_attention, Python's sorted).

The functions are plain so that the mutation test can run them against
deliberately broken builds of the oracle in a separate process.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split(":", 1)
            vals[k.strip()] = [float(x) for x in v.split()]
    return vals


def _bf(x):
    return W.to_bf16_bits(np.asarray(x, dtype=np.float32))


# --------------------------------------------------------------------------
# indexer
# --------------------------------------------------------------------------
def pin_indexer_worked_example():
    """tests/golden/indexer_worked_example.txt (exo #2539 Prefill, indexer)."""
    g = _read_golden("indexer_worked_example.txt")
    Hi, Di, q0 = int(g["Hi"][0]), int(g["Di"][0]), int(g["q_start"][0])
    qI = _bf(np.array(g["qI"]).reshape(2, Hi, Di))
    kI = _bf(np.array(g["kI"]).reshape(3, Di))
    w = np.array(g["w"], dtype=np.float32).reshape(2, Hi)
    S = oracle.indexer_scores(qI, kI, w, q0)
    want = np.array(g["S"], dtype=np.float32).reshape(2, 3)
    assert np.array_equal(S, want), (S, want)
    for k in (1, 2, 3):
        idx, cnt = oracle.topk_select(S, q0 + np.arange(2), k)
        assert np.array_equal(idx.ravel(), np.array(g["topk%d_idx" % k], dtype=np.int32)), (k, idx)
        assert np.array_equal(cnt, np.array(g["topk%d_count" % k], dtype=np.int32)), (k, cnt)


def pin_indexer_exact_rational():
    """Brute force in exact rational arithmetic on tiny random integer inputs:
    the fp32 score must be the exact value rounded once to float32."""
    rng = np.random.default_rng(7)
    for trial in range(4):
        L, N, Hi, Di, q0 = 3, 7, 3, 5, 4
        qI = rng.integers(-8, 9, size=(L, Hi, Di))
        kI = rng.integers(-8, 9, size=(N, Di))
        w = rng.choice([0.5, 1.0, 2.0, -1.0, 0.25], size=(L, Hi)).astype(np.float32)
        S = oracle.indexer_scores(_bf(qI), _bf(kI), w, q0)
        for i in range(L):
            for j in range(N):
                if j > q0 + i:
                    assert S[i, j] == -np.inf
                    continue
                exact = Fraction(0)
                for h in range(Hi):
                    dot = sum(int(qI[i, h, d]) * int(kI[j, d]) for d in range(Di))
                    exact += Fraction(float(w[i, h])) * max(dot, 0)
                assert S[i, j] == np.float32(float(exact)), (i, j, S[i, j], exact)


def pin_indexer_one_hot_closed_form():
    """qI[i,h] = c_h * e_{d_h}  =>  S[i,j] = sum_h w_h relu(c_h kI[j,d_h])."""
    rng = np.random.default_rng(8)
    L, N, Hi, Di, q0 = 4, 9, 4, 6, 5
    d_h = rng.integers(0, Di, size=(L, Hi))
    c_h = rng.choice([-2.0, -1.0, 1.0, 3.0], size=(L, Hi))
    qI = np.zeros((L, Hi, Di))
    for i in range(L):
        for h in range(Hi):
            qI[i, h, d_h[i, h]] = c_h[i, h]
    kI = rng.integers(-5, 6, size=(N, Di)).astype(np.float64)
    w = rng.choice([0.5, 1.0, 2.0], size=(L, Hi)).astype(np.float32)
    S = oracle.indexer_scores(_bf(qI), _bf(kI), w, q0)
    for i in range(L):
        for j in range(q0 + i + 1):
            want = sum(w[i, h] * max(c_h[i, h] * kI[j, d_h[i, h]], 0.0) for h in range(Hi))
            assert S[i, j] == np.float32(want), (i, j, S[i, j], want)


def pin_indexer_relu_mask_linearity():
    """relu clips negative dot products to 0; the mask is -inf exactly past the
    query's position (diagonal included); the score is linear in w and
    invariant under a joint permutation of the heads."""
    rng = np.random.default_rng(9)
    L, N, Hi, Di, q0 = 5, 12, 4, 8, 7
    kI = np.abs(rng.integers(1, 5, size=(N, Di)))
    qI_neg = -np.abs(rng.integers(1, 5, size=(L, Hi, Di)))       # every q.k < 0
    w = rng.choice([0.5, 1.0, 2.0], size=(L, Hi)).astype(np.float32)
    S = oracle.indexer_scores(_bf(qI_neg), _bf(kI), w, q0)
    for i in range(L):
        assert np.all(S[i, : q0 + i + 1] == 0.0), S[i]
        assert np.all(S[i, q0 + i + 1:] == -np.inf), S[i]
    qI = rng.integers(-8, 9, size=(L, Hi, Di))
    S1 = oracle.indexer_scores(_bf(qI), _bf(kI), w, q0)
    S2 = oracle.indexer_scores(_bf(qI), _bf(kI), 2 * w, q0)
    S3 = oracle.indexer_scores(_bf(qI), _bf(kI), -w, q0)
    perm = rng.permutation(Hi)
    S4 = oracle.indexer_scores(_bf(qI[:, perm]), _bf(kI), np.ascontiguousarray(w[:, perm]), q0)
    vis = np.isfinite(S1)
    assert np.array_equal(vis, np.arange(N)[None, :] <= (q0 + np.arange(L))[:, None])
    assert np.array_equal(S2[vis], 2 * S1[vis])
    assert np.array_equal(S3[vis], -S1[vis])
    assert np.array_equal(S4, S1)


# --------------------------------------------------------------------------
# top-k
# --------------------------------------------------------------------------
def _brute_topk(srow, p, k):
    keys = list(range(p + 1))
    if p + 1 <= k:
        sel = keys
    else:
        sel = sorted(keys, key=lambda j: (-float(srow[j]), j))[:k]
    sel = sorted(sel)
    return sel + [-1] * (k - len(sel)), len(sel)


def pin_topk_brute_force():
    """Python's sorted() on (-score, key) over tiny rows, with many ties."""
    rng = np.random.default_rng(10)
    for trial in range(30):
        N = int(rng.integers(1, 40))
        k = int(rng.integers(1, 12))
        nrows = 6
        S = rng.integers(0, 4, size=(nrows, N)).astype(np.float32)     # heavy ties
        if trial % 3 == 1:
            S = rng.standard_normal((nrows, N)).astype(np.float32)
        if trial % 3 == 2:
            S = -np.abs(S) - 1.0                                      # all negative
        pos = rng.integers(0, N, size=nrows)
        idx, cnt = oracle.topk_select(S, pos, k)
        for r in range(nrows):
            want, c = _brute_topk(S[r], int(pos[r]), k)
            assert list(idx[r]) == want, (trial, r, list(idx[r]), want)
            assert cnt[r] == c


def pin_topk_boundary_rule():
    """p+1 == top_k takes every earlier key regardless of scores; p+1 ==
    top_k+1 drops exactly the single worst key (ties to the higher index)."""
    k = 8
    S = np.zeros((2, 16), dtype=np.float32)
    S[0, :8] = [-5, -4, -3, -2, -1, -6, -7, -8]
    S[1, :9] = [3, 3, 3, 3, 3, 3, 3, 3, 3]
    idx, cnt = oracle.topk_select(S, np.array([7, 8]), k)
    assert list(idx[0]) == list(range(8)) and cnt[0] == 8
    assert list(idx[1]) == list(range(8)) and cnt[1] == 8        # key 8 loses the tie
    S[1, 0] = 2.0                                                # now key 0 is the worst
    idx, cnt = oracle.topk_select(S, np.array([7, 8]), k)
    assert list(idx[1]) == list(range(1, 9))


def pin_topk_invariants_tiny():
    """On the tiny workload: ascending, inside the causal range, count =
    min(p+1, top_k), every kept score >= every dropped score, and among equal
    scores at the boundary the kept keys have the lower indices."""
    cfg = W.PREFILL["tiny"]
    d = W.make_prefill(cfg)
    S = oracle.indexer_scores(d["qI"], d["kI"], d["w"], cfg.q_start)
    pos = cfg.q_start + np.arange(cfg.L)
    idx, cnt = oracle.topk_select(S, pos, cfg.shape.top_k)
    for r in range(cfg.L):
        p = int(pos[r])
        c = int(cnt[r])
        sel = idx[r, :c]
        assert c == min(p + 1, cfg.shape.top_k)
        assert np.all(idx[r, c:] == -1)
        assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] <= p
        mask = np.zeros(p + 1, bool)
        mask[sel] = True
        kept, dropped = S[r, : p + 1][mask], S[r, : p + 1][~mask]
        if dropped.size:
            assert kept.min() >= dropped.max()
            t = kept.min()
            if dropped.max() == t:
                assert np.flatnonzero(mask & (S[r, : p + 1] == t)).max() < \
                    np.flatnonzero(~mask & (S[r, : p + 1] == t)).min()


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def pin_attention_worked_example():
    """tests/golden/attention_worked_example.txt (closed form)."""
    g = _read_golden("attention_worked_example.txt")
    q = _bf(np.array(g["q"]).reshape(1, 1, 3))
    kv = _bf(np.array(g["kv"]).reshape(3, 3))
    idx = np.array([g["idx"]], dtype=np.int32)
    cnt = np.array([int(g["count"][0])], dtype=np.int32)
    out, lse = oracle.sparse_mla_attn(q, kv, idx, cnt, 2, 1.0 / 16, want_lse=True)
    assert np.allclose(out.ravel(), g["out"], rtol=0, atol=1e-15), out
    assert abs(lse[0, 0] - g["lse"][0]) < 1e-14, lse


def _sdpa(q, kv, mask, Dl, scale):
    import torch
    qf = torch.from_numpy(W.bf16_bits_to_f32(q).astype(np.float64))          # [L,H,D]
    kf = torch.from_numpy(W.bf16_bits_to_f32(kv).astype(np.float64))         # [N,D]
    vf = kf[:, :Dl]
    L, H, D = qf.shape
    qh = qf.permute(1, 0, 2).contiguous()                                      # [H,L,D]
    kh = kf.unsqueeze(0).expand(H, -1, -1).contiguous()
    vh = vf.unsqueeze(0).expand(H, -1, -1).contiguous()
    m = torch.from_numpy(mask).unsqueeze(0).expand(H, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=m, scale=scale)
    return o.permute(1, 0, 2).numpy()                                          # [L,H,Dl]


def pin_attention_dense_equals_sdpa():
    """When every query keeps every earlier key (top_k >= p+1), the chunk is
    textbook causal attention: torch's SDPA in float64 with a j <= p mask."""
    for name in ("tiny_dense", "glm_small_first"):
        cfg = W.PREFILL[name]
        d = W.make_prefill(cfg)
        rows = np.arange(cfg.L) if cfg.L <= 64 else W.sample_rows(cfg.L, 16)
        idx, cnt, out = oracle.prefill_chunk(d, cfg.shape, cfg.q_start, rows=rows)
        pos = cfg.q_start + rows
        assert np.array_equal(cnt, pos + 1)
        mask = np.arange(cfg.N)[None, :] <= pos[:, None]
        ref = _sdpa(d["q"][rows], d["kv"], mask, cfg.shape.d_latent, cfg.shape.softmax_scale)
        err = np.abs(out - ref).max() / np.abs(ref).max()
        assert err < 1e-12, (name, err)


def pin_attention_sparse_equals_masked_sdpa():
    """Sparse attention over a selection equals dense attention with every
    unselected key masked out (torch SDPA, float64); selection order is free."""
    rng = np.random.default_rng(12)
    cfg = W.PREFILL["tiny"]
    d = W.make_prefill(cfg)
    L, N, k = cfg.L, cfg.N, cfg.shape.top_k
    idx = np.full((L, k), -1, np.int32)
    cnt = rng.integers(1, k + 1, size=L).astype(np.int32)
    mask = np.zeros((L, N), bool)
    for i in range(L):
        sel = rng.choice(N, size=cnt[i], replace=False)          # unsorted on purpose
        idx[i, : cnt[i]] = sel
        mask[i, sel] = True
    out = oracle.sparse_mla_attn(d["q"], d["kv"], idx, cnt, cfg.shape.d_latent, cfg.shape.softmax_scale)
    ref = _sdpa(d["q"], d["kv"], mask, cfg.shape.d_latent, cfg.shape.softmax_scale)
    err = np.abs(out - ref).max() / np.abs(ref).max()
    assert err < 1e-12, err


def pin_attention_closed_forms():
    """All selected rows equal -> out = that row's value part; q = 0 -> out =
    mean of the selected value rows and lse = log(count); one key -> its
    value; the output does not depend on the order of the selection."""
    rng = np.random.default_rng(13)
    H, Dl, Dr, N, k = 3, 8, 4, 20, 6
    D = Dl + Dr
    kv = _bf(rng.standard_normal((N, D)))
    q = _bf(rng.standard_normal((2, H, D)) * 3)
    sel = rng.choice(N, size=k, replace=False).astype(np.int32)
    idx = np.stack([sel, sel])
    cnt = np.array([k, 1], np.int32)
    kvf = W.bf16_bits_to_f32(kv).astype(np.float64)
    # one key
    out = oracle.sparse_mla_attn(q, kv, idx, cnt, Dl, 1.0 / 16)
    assert np.allclose(out[1], kvf[sel[0], :Dl][None, :], rtol=0, atol=0)
    # equal rows
    kv_eq = np.tile(kv[sel[0]], (N, 1))
    out = oracle.sparse_mla_attn(q, kv_eq, idx, cnt, Dl, 1.0 / 16)
    assert np.allclose(out, kvf[sel[0], :Dl][None, None, :], rtol=0, atol=1e-15)
    # zero query
    q0 = np.zeros_like(q)
    out, lse = oracle.sparse_mla_attn(q0, kv, idx, cnt, Dl, 1.0 / 16, want_lse=True)
    assert np.allclose(out[0], kvf[sel, :Dl].mean(0)[None, :], rtol=0, atol=1e-15)
    assert np.allclose(lse[0], math.log(k), rtol=0, atol=1e-15)
    assert np.allclose(lse[1], 0.0, rtol=0, atol=1e-15)
    # order of the selection
    out_a = oracle.sparse_mla_attn(q, kv, idx, cnt, Dl, 1.0 / 16)
    idx_b = idx.copy()
    idx_b[0] = sel[rng.permutation(k)]
    out_b = oracle.sparse_mla_attn(q, kv, idx_b, cnt, Dl, 1.0 / 16)
    assert np.allclose(out_a, out_b, rtol=0, atol=1e-14)


def pin_attention_scale_and_rope_part():
    """The rope columns enter the score but not the value; the scale divides
    the dot product: moving a factor 2 from the scale into q is a no-op."""
    rng = np.random.default_rng(14)
    H, Dl, Dr, N = 2, 8, 8, 10
    kv = rng.standard_normal((N, Dl + Dr))
    kv[:, Dl:] = 0.0
    q = rng.standard_normal((1, H, Dl + Dr))
    sel = np.arange(N, dtype=np.int32)[None, :]
    cnt = np.array([N], np.int32)
    a = oracle.sparse_mla_attn(_bf(q), _bf(kv), sel, cnt, Dl, 1.0 / 16)
    q2 = q.copy()
    q2[..., Dl:] = 100.0                       # rope part of q meets zero keys
    b = oracle.sparse_mla_attn(_bf(q2), _bf(kv), sel, cnt, Dl, 1.0 / 16)
    assert np.allclose(a, b, rtol=0, atol=1e-14)
    c = oracle.sparse_mla_attn(_bf(q * 2), _bf(kv), sel, cnt, Dl, 1.0 / 32)
    assert np.allclose(a, c, rtol=0, atol=1e-14)
    # a key whose rope part alone makes it dominant
    kv3 = np.zeros((3, Dl + Dr))
    kv3[0, :Dl] = 1.0
    kv3[1, :Dl] = -1.0
    kv3[1, Dl:] = 1.0
    q3 = np.zeros((1, 1, Dl + Dr))
    q3[..., Dl:] = 64.0                        # s_1 = 8*64/16 = 32, s_0 = 0
    out = oracle.sparse_mla_attn(_bf(q3), _bf(kv3), np.array([[0, 1]], np.int32),
                                 np.array([2], np.int32), Dl, 1.0 / 16)
    p1 = 1.0 / (1.0 + math.exp(-32.0))
    assert np.allclose(out[0, 0], (1 - p1) * 1.0 + p1 * -1.0, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# chunk and decode compositions
# --------------------------------------------------------------------------
def pin_chunk_composition_matches_stages():
    """The chunk runs the stages in the pages' order: its selection equals
    brute-force selection over the indexer's scores (dense rule below top_k),
    and its output equals masked SDPA over that selection."""
    cfg = W.PREFILL["tiny"]
    d = W.make_prefill(cfg)
    idx, cnt, out = oracle.prefill_chunk(d, cfg.shape, cfg.q_start)
    S = oracle.indexer_scores(d["qI"], d["kI"], d["w"], cfg.q_start)
    mask = np.zeros((cfg.L, cfg.N), bool)
    for i in range(cfg.L):
        want, c = _brute_topk(S[i], cfg.q_start + i, cfg.shape.top_k)
        assert list(idx[i]) == want and cnt[i] == c
        mask[i, idx[i, :c]] = True
    ref = _sdpa(d["q"], d["kv"], mask, cfg.shape.d_latent, cfg.shape.softmax_scale)
    assert np.abs(out - ref).max() / np.abs(ref).max() < 1e-12


def pin_decode_dense_sequences_equal_sdpa():
    """A decode sequence whose context fits in top_k is plain attention of its
    last position over its whole cache."""
    cfg = W.DECODE["tiny_decode"]
    d = W.make_decode(cfg)
    idx, cnt, out = oracle.decode_step(d, cfg.shape)
    off = d["row_off"]
    for b, c in enumerate(cfg.ctx):
        assert cnt[b] == min(c, cfg.shape.top_k)
        if c > cfg.shape.top_k:
            continue
        kvb = d["kv"][off[b]: off[b + 1]]
        ref = _sdpa(d["q"][b: b + 1], kvb, np.ones((1, c), bool), cfg.shape.d_latent,
                    cfg.shape.softmax_scale)
        assert np.abs(out[b] - ref[0]).max() / np.abs(ref).max() < 1e-12, b


def pin_decode_sparse_sequences_follow_brute_force():
    """A decode sequence with a context longer than top_k keeps the
    brute-force top_k of its exact scores over its own cache."""
    cfg = W.DECODE["tiny_decode"]
    d = W.make_decode(cfg)
    idx, cnt, out = oracle.decode_step(d, cfg.shape)
    off = d["row_off"]
    for b, c in enumerate(cfg.ctx):
        if c <= cfg.shape.top_k:
            continue
        S = oracle.indexer_scores(d["qI"][b: b + 1], d["kI"][off[b]: off[b + 1]], d["w"][b: b + 1], c - 1)
        want, n = _brute_topk(S[0], c - 1, cfg.shape.top_k)
        assert list(idx[b]) == want and cnt[b] == n, b
        mask = np.zeros((1, c), bool)
        mask[0, idx[b, :n]] = True
        ref = _sdpa(d["q"][b: b + 1], d["kv"][off[b]: off[b + 1]], mask, cfg.shape.d_latent,
                    cfg.shape.softmax_scale)
        assert np.abs(out[b] - ref[0]).max() / np.abs(ref).max() < 1e-12, b


# --------------------------------------------------------------------------
# upstream cache write (pipeline trace sections 4 and 5)
# --------------------------------------------------------------------------
def _f(bits):
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def _half_ulp_bf16(x):
    """Half a bf16 unit in the last place at |x| (normal range)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, 1e-30)))
    return np.ldexp(1.0, (e - 8).astype(int))


def _cw(shape, T, N, pos, kv_a=None, norm_w=None, eps=0.0, q=None, qI=None, kI_new=None,
        d_idx_rope=None, theta=10000.0):
    """Run the oracle's cache write on zero caches; missing operands are zeros."""
    Dqk = shape.d_qk
    kv_a = np.zeros((T, Dqk), np.uint16) if kv_a is None else kv_a
    norm_w = np.ones(shape.d_latent, np.float32) if norm_w is None else norm_w
    kI_new = np.zeros((T, shape.d_idx), np.uint16) if kI_new is None else kI_new
    return oracle.cache_write(kv_a, norm_w, eps, np.asarray(pos, np.int64),
                              np.zeros((N, Dqk), np.uint16), kI_new,
                              np.zeros((N, shape.d_idx), np.uint16), q, qI, shape=shape,
                              d_idx_rope=shape.d_rope if d_idx_rope is None else d_idx_rope,
                              theta=theta)


def pin_rope_position_zero_is_identity():
    """At position 0 every rotation angle is 0: q, qI and the key rows keep
    their bits."""
    cfg = W.CACHE_WRITE["tiny"]
    d = W.make_cache_write(cfg)
    sh = cfg.shape
    kv, kI, q, qI = oracle.cache_write(d["kv_a"][:3], d["norm_w"], cfg.eps, np.zeros(3, np.int64),
                                      d["kv_cache"], d["kI_new"][:3], d["kI_cache"], d["q"][:3],
                                      d["qI"][:3], shape=sh, d_idx_rope=cfg.d_idx_rope, theta=cfg.theta)
    assert np.array_equal(q, d["q"][:3]) and np.array_equal(qI, d["qI"][:3])
    assert np.array_equal(kv[0, sh.d_latent:], d["kv_a"][2, sh.d_latent:])   # last write wins
    assert np.array_equal(kI[0], d["kI_new"][2])


def pin_rope_interleaved_pair_closed_form():
    """NORM flavour (pipeline trace section 5): a one-hot x[2i] = 1 at
    position p comes out as (cos a, sin a) in columns 2i, 2i+1 and zero
    elsewhere, a = p * theta^(-2i/d); each value is the exact one rounded
    once to bf16."""
    sh = W.TINY
    d, theta = sh.d_rope, 10000.0
    for i, p in ((0, 5), (1, 7), (3, 11), (d // 2 - 1, 40000)):
        q = np.zeros((1, sh.n_heads, sh.d_qk), np.uint16)
        q[0, 2, sh.d_latent + 2 * i] = np.uint16(0x3F80)   # 1.0
        _, _, qo, _ = _cw(sh, 1, 4, [p], q=q, theta=theta)
        got = _f(qo[0, 2, sh.d_latent:])
        a = p * theta ** (-2.0 * i / d)
        want = np.zeros(d)
        want[2 * i], want[2 * i + 1] = math.cos(a), math.sin(a)
        assert np.all(np.abs(got - want) <= _half_ulp_bf16(want) * 1.0000001), (i, p, got, want)
        assert np.count_nonzero(got[np.arange(d) // 2 != i]) == 0
        assert not np.any(_f(qo[0, [0, 1, 3]])) and not np.any(_f(qo[0, 2, :sh.d_latent]))


def pin_rope_frequency_ladder():
    """Recovered from one-hot inputs at p = 1, pair i turns by theta^(-2i/d):
    pair 0 by exactly 1 radian and each next pair by theta^(-2/d) times the
    previous angle (the indexer rope over d_idx_rope = 2 * d_rope included)."""
    sh = W.TINY
    theta = 500.0
    for width, which in ((sh.d_rope, "q"), (2 * sh.d_rope, "qI")):
        ang = []
        for i in range(width // 2):
            if which == "q":
                x = np.zeros((1, sh.n_heads, sh.d_qk), np.uint16)
                x[0, 0, sh.d_latent + 2 * i] = np.uint16(0x3F80)   # 1.0
                _, _, out, _ = _cw(sh, 1, 2, [1], q=x, theta=theta)
                o = _f(out[0, 0, sh.d_latent + 2 * i: sh.d_latent + 2 * i + 2])
            else:
                x = np.zeros((1, sh.n_idx_heads, sh.d_idx), np.uint16)
                x[0, 1, 2 * i] = np.uint16(0x3F80)   # 1.0
                _, _, _, out = _cw(sh, 1, 2, [1], qI=x, theta=theta, d_idx_rope=width)
                o = _f(out[0, 1, 2 * i: 2 * i + 2])
            ang.append(math.atan2(o[1], o[0]))
        ang = np.array(ang)
        assert abs(ang[0] - 1.0) < 4e-3, ang[0]
        ratio = ang[1:] / ang[:-1]
        assert np.all(np.abs(ratio - theta ** (-2.0 / width)) < 0.01), (which, ratio)


def pin_rope_rotation_invariants():
    """A rotation keeps each pair's length and composes additively in the
    position: rope(rope(x, a), b) = rope(x, a + b) (up to the two extra bf16
    roundings)."""
    cfg = W.CACHE_WRITE["tiny"]
    d = W.make_cache_write(cfg)
    sh = cfg.shape
    q0 = d["q"][:4]
    pa, pb = np.array([3, 100, 2047, 12345]), np.array([9, 1, 4000, 7])
    _, _, qa, _ = _cw(sh, 4, 1, pa, q=q0)
    _, _, qab, _ = _cw(sh, 4, 1, pb, q=qa)
    _, _, qs, _ = _cw(sh, 4, 1, pa + pb, q=q0)
    x0 = _f(q0[..., sh.d_latent:]).reshape(4, sh.n_heads, -1, 2)
    xa = _f(qa[..., sh.d_latent:]).reshape(4, sh.n_heads, -1, 2)
    n0, na = np.hypot(x0[..., 0], x0[..., 1]), np.hypot(xa[..., 0], xa[..., 1])
    assert np.all(np.abs(na - n0) <= 2.0 ** -7 * n0 + 1e-30)
    # three bf16 roundings of at most 2^-8 of the pair's length each
    tol = 2.0 ** -6 * np.repeat(n0, 2, axis=-1)
    diff = np.abs(_f(qab[..., sh.d_latent:]) - _f(qs[..., sh.d_latent:]))
    assert np.all(diff <= tol + 1e-30), float((diff - tol).max())


def pin_rmsnorm_closed_forms():
    """RMSNorm (x / sqrt(mean(x^2) + eps) * weight, after the split, section
    4): constant rows, alternating rows, an eps that doubles the RMS, and
    invariance under a power-of-two scaling of x."""
    sh = W.TINY
    Dl, Dqk = sh.d_latent, sh.d_qk
    wv = _f(_bf(np.linspace(-2.0, 2.0, Dl, dtype=np.float32))).astype(np.float32)
    x = np.zeros((4, Dqk), np.float32)
    x[0, :Dl] = 3.0                                   # mean(x^2) = 9: y = w
    x[1, :Dl] = np.where(np.arange(Dl) % 2, -0.5, 0.5)  # y = +-w
    x[2, :Dl] = 1.0                                   # with eps = 3: y = w / 2
    x[3, :Dl] = 0.375 * np.arange(1, Dl + 1)
    kv_a = _bf(x)
    kv0, _, _, _ = _cw(sh, 4, 4, [0, 1, 2, 3], kv_a=kv_a, norm_w=wv, eps=0.0)
    kv3, _, _, _ = _cw(sh, 4, 4, [0, 1, 2, 3], kv_a=kv_a, norm_w=wv, eps=3.0)
    assert np.array_equal(kv0[0, :Dl], _bf(wv))
    assert np.array_equal(kv0[1, :Dl], _bf(np.where(np.arange(Dl) % 2, -wv, wv)))
    assert np.array_equal(kv3[2, :Dl], _bf(wv / 2))
    kv_a4 = kv_a.copy()
    kv_a4[3, :Dl] = _bf(4.0 * _f(kv_a[3, :Dl]))
    kv4, _, _, _ = _cw(sh, 4, 4, [0, 1, 2, 3], kv_a=kv_a4, norm_w=wv, eps=0.0)
    assert np.array_equal(kv4[3, :Dl], kv0[3, :Dl])
    # the exact value, rounded once
    r = _f(kv_a[3, :Dl])
    want = r / math.sqrt(np.mean(r * r)) * wv
    got = _f(kv0[3, :Dl])
    assert np.all(np.abs(got - want) <= _half_ulp_bf16(want) * 1.0000001)


def pin_cache_write_rows_and_layout():
    """Only rows named by in-range positions change; a row holds
    [normed kv_cmpr | roped k_pe]; the indexer row ropes its leading
    d_idx_rope columns and copies the rest; the query's latent columns stay."""
    cfg = W.CACHE_WRITE["tiny"]
    d = W.make_cache_write(cfg)
    sh = cfg.shape
    kv, kI, q, qI = oracle.cache_write(d["kv_a"], d["norm_w"], cfg.eps, d["pos"], d["kv_cache"],
                                      d["kI_new"], d["kI_cache"], d["q"], d["qI"], shape=sh,
                                      d_idx_rope=cfg.d_idx_rope, theta=cfg.theta)
    good = (d["pos"] >= 0) & (d["pos"] < cfg.N)
    assert (~good).sum() == 2
    hit = np.zeros(cfg.N, bool)
    hit[d["pos"][good]] = True
    assert np.array_equal(kv[~hit], d["kv_cache"][~hit]) and np.array_equal(kI[~hit], d["kI_cache"][~hit])
    assert np.array_equal(q[..., :sh.d_latent], d["q"][..., :sh.d_latent])
    assert np.array_equal(kI[d["pos"][good], cfg.d_idx_rope:], d["kI_new"][good, cfg.d_idx_rope:])
    assert np.array_equal(qI[..., cfg.d_idx_rope:], d["qI"][..., cfg.d_idx_rope:])
    # the rope part of row pos[t] equals q's rotation of the same vector at pos[t]
    t = int(np.flatnonzero(good)[0])
    qq = np.zeros((1, sh.n_heads, sh.d_qk), np.uint16)
    qq[0, 1, sh.d_latent:] = d["kv_a"][t, sh.d_latent:]
    _, _, qo, _ = _cw(sh, 1, 1, [d["pos"][t]], q=qq, theta=cfg.theta)
    assert np.array_equal(kv[d["pos"][t], sh.d_latent:], qo[0, 1, sh.d_latent:])
    # and the latent part does not depend on the position
    kv2, _, _, _ = oracle.cache_write(d["kv_a"][t:t + 1], d["norm_w"], cfg.eps, np.array([5]),
                                      d["kv_cache"], None, None, None, None, shape=sh,
                                      d_idx_rope=cfg.d_idx_rope, theta=cfg.theta)
    assert np.array_equal(kv2[5, :sh.d_latent], kv[d["pos"][t], :sh.d_latent])


# --------------------------------------------------------------------------
# router selection (pipeline trace section 8a)
# --------------------------------------------------------------------------
def _router_brute(logits, bias, k, scale):
    """Independent ranking with Python's sort on (score desc, expert asc);
    the float32 probability is the exact sigmoid rounded once (math.exp in
    double, then numpy's float32 rounding) and the score a float32 sum."""
    T, E = logits.shape
    ids = np.empty((T, k), np.int64)
    wts = np.empty((T, k))
    for t in range(T):
        p = np.array([1.0 / (1.0 + math.exp(-float(x))) for x in logits[t]]).astype(np.float32)
        sc = p + bias                                     # float32 + float32
        order = sorted(range(E), key=lambda e: (-float(sc[e]), e))[:k]
        ids[t] = order
        tot = sum(float(p[e]) for e in order)
        wts[t] = [float(p[e]) / max(tot, oracle.ROUTER_MIN_SUM) * scale for e in order]
    return ids, wts


def pin_router_brute_force():
    """Selections on random and on heavily tied inputs equal a plain sort."""
    for name in ("small", "small_ties", "glm_ties"):
        cfg = W.ROUTER[name]
        d = W.make_router(cfg)
        ids, wts = oracle.router_topk(d["logits"], d["bias"], cfg.k, cfg.scale)
        bi, bw = _router_brute(d["logits"], d["bias"], cfg.k, cfg.scale)
        assert np.array_equal(ids, bi), name
        assert np.allclose(wts, bw, rtol=1e-12, atol=0), name


def pin_router_closed_forms():
    """Equal logits: experts 0..k-1 (ties to the lower index), each weighted
    scale/k.  A large bias selects an expert first without entering its
    weight.  Weights of a normalised selection sum to the scale."""
    E, k, sc = 16, 4, 2.5
    ids, wts = oracle.router_topk(np.zeros((1, E), np.float32), np.zeros(E, np.float32), k, sc)
    assert list(ids[0]) == [0, 1, 2, 3] and np.allclose(wts, sc / k, rtol=1e-15)
    lg = np.zeros((1, E), np.float32)
    lg[0, E - 1] = -4.0
    b = np.zeros(E, np.float32)
    b[E - 1] = 10.0
    ids, wts = oracle.router_topk(lg, b, k, sc)
    assert list(ids[0]) == [E - 1, 0, 1, 2]
    p = float(np.float32(1.0 / (1.0 + math.exp(4.0))))
    assert abs(wts[0, 0] - p / (p + 1.5) * sc) < 1e-12 and abs(wts[0, 1] - 0.5 / (p + 1.5) * sc) < 1e-12
    cfg = W.ROUTER["small"]
    d = W.make_router(cfg)
    _, wts = oracle.router_topk(d["logits"], d["bias"], cfg.k, cfg.scale)
    assert np.allclose(wts.sum(axis=1), cfg.scale, rtol=1e-12)


def pin_router_weight_clamp():
    """Probabilities far below the clamp: the weight sum is held at 6.1e-5,
    so the weights are p / 6.1e-5 * scale rather than summing to the scale."""
    E, k, sc = 32, 8, 2.5
    lg = np.full((1, E), -30.0, np.float32)
    ids, wts = oracle.router_topk(lg, np.zeros(E, np.float32), k, sc)
    p = float(np.float32(1.0 / (1.0 + math.exp(30.0))))
    assert list(ids[0]) == list(range(k))
    assert np.allclose(wts, p / 6.1e-5 * sc, rtol=1e-12)


def pin_router_sigmoid_symmetry():
    """sigmoid(x) + sigmoid(-x) = 1 (each rounded once to float): with equal
    bias, expert 0 at +x and expert 1 at -x, k = 2, the weights are the two
    probabilities over their sum of 1 (to float rounding)."""
    for x in (0.25, 1.0, 3.0, 7.5):
        lg = np.array([[x, -x]], np.float32)
        ids, wts = oracle.router_topk(lg, np.zeros(2, np.float32), 2, 1.0)
        assert list(ids[0]) == [0, 1]
        assert abs(wts[0].sum() - 1.0) < 1e-15 and abs(wts[0, 0] + wts[0, 1] - 1.0) < 1e-15
        pp = 1.0 / (1.0 + math.exp(-x))
        assert abs(wts[0, 0] - pp) < 2.0 ** -24 * 2 and abs(wts[0, 1] - (1 - pp)) < 2.0 ** -24 * 2


# --------------------------------------------------------------------------
# downstream projections (pipeline trace section 6, build_attn)
# --------------------------------------------------------------------------
def pin_up_proj_identity_and_single_rounding():
    """An identity up-projection returns the attention output rounded once to
    bf16; a row of two ones adds the two bf16-rounded inputs and rounds the
    sum once (1 + 2^-8 + 2^-10 rounds to 1 + 2^-7; plus 2^-8 the sum is a
    bf16 midpoint that goes to the even 1 + 2^-6, where the unrounded sum
    would give 1 + 2^-7)."""
    T, H, Dl, Dv = 3, 2, 64, 32
    rng = np.random.default_rng(7)
    o = rng.standard_normal((T, H, Dl)).astype(np.float32)
    wv = np.zeros((H, Dv, Dl), np.uint16)
    for h in range(H):
        for j in range(Dv):
            wv[h, j, j] = 0x3F80
    out = oracle.value_up_proj(o, wv)
    assert np.array_equal(out, W.to_bf16_bits(o[..., :Dv]))
    o2 = np.zeros((1, 1, Dl), np.float32)
    o2[0, 0, 0] = 1 + 2.0 ** -8 + 2.0 ** -10
    o2[0, 0, 1] = 2.0 ** -8
    w2 = np.zeros((1, 1, Dl), np.uint16)
    w2[0, 0, 0] = w2[0, 0, 1] = 0x3F80
    got = float(W.bf16_bits_to_f32(oracle.value_up_proj(o2, w2))[0, 0, 0])
    assert got == 1 + 2.0 ** -6, got


def pin_projections_match_numpy():
    """Both projections on random bf16 data equal numpy's float64 matmul of
    the decoded operands (the up-projection within its final rounding)."""
    rng = np.random.default_rng(8)
    T, H, Dl, Dv, hid = 5, 3, 64, 32, 48
    o = rng.standard_normal((T, H, Dl)).astype(np.float32)
    wv = W.to_bf16_bits(rng.standard_normal((H, Dv, Dl)).astype(np.float32))
    out = oracle.value_up_proj(o, wv)
    ob = _f(W.to_bf16_bits(o))
    ref = np.einsum("thc,hjc->thj", ob, _f(wv))
    got = _f(out)
    assert np.all(np.abs(got - ref) <= _half_ulp_bf16(ref) * 1.0000001 + 1e-30)
    x = W.to_bf16_bits(rng.standard_normal((T, H * Dv)).astype(np.float32))
    wo = W.to_bf16_bits(rng.standard_normal((hid, H * Dv)).astype(np.float32))
    y = oracle.o_proj(x, wo)
    ref = _f(x) @ _f(wo).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    rows = np.array([4, 0, 2])
    assert np.array_equal(oracle.o_proj(x, wo, rows), y[rows])


def pin_o_proj_one_hot_rows():
    """Output row n of a one-hot weight picks input column n's value."""
    rng = np.random.default_rng(9)
    T, K, N = 4, 64, 16
    x = W.to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    wo = np.zeros((N, K), np.uint16)
    cols = rng.choice(K, size=N, replace=False)
    wo[np.arange(N), cols] = 0x3F80
    y = oracle.o_proj(x, wo)
    assert np.array_equal(y, _f(x)[:, cols])


# --------------------------------------------------------------------------
# dense masked attention, non-absorbed form
# --------------------------------------------------------------------------
def _dense_absorbed_pair(rng, L, N, H, Dl, Dn, Dr, Dv, q_start, top_k, scale):
    """Both forms of one attention on integer-valued data: latent rows, rope
    keys, projection weights and queries are small integers, so every bf16
    input of both forms (the up-projected keys and values, the absorbed
    query) is exact and the forms must agree to double rounding."""
    lat = rng.integers(-2, 3, size=(N, Dl))
    rope = rng.integers(-2, 3, size=(N, Dr))
    wkb = rng.integers(-1, 2, size=(H, Dn, Dl))
    wvb = rng.integers(-1, 2, size=(H, Dv, Dl))
    qn = rng.integers(-1, 2, size=(L, H, Dn))
    qp = rng.integers(-1, 2, size=(L, H, Dr))
    kn = np.einsum("hdc,jc->jhd", wkb, lat)
    v = np.einsum("hec,jc->jhe", wvb, lat)
    qabs = np.einsum("ihd,hdc->ihc", qn, wkb)
    assert max(np.abs(kn).max(), np.abs(v).max(), np.abs(qabs).max()) <= 256   # exact in bf16
    kv = _bf(np.concatenate([lat, rope], axis=1))
    q_abs = _bf(np.concatenate([qabs, qp], axis=2))
    q_dense = _bf(np.concatenate([qn, qp], axis=2))
    kvb = _bf(np.concatenate([kn, v], axis=2))
    S = rng.standard_normal((L, N)).astype(np.float32)
    pos = q_start + np.arange(L)
    S[np.arange(N)[None, :] > pos[:, None]] = -np.inf
    idx, cnt = oracle.topk_select(S, pos, top_k)
    sparse = oracle.sparse_mla_attn(q_abs, kv, idx, cnt, Dl, scale)
    expected = np.einsum("ihc,hec->ihe", sparse, wvb.astype(np.float64))
    mask = oracle.selection_mask(idx, cnt, N, q_start)
    dense = oracle.dense_masked_attn(q_dense, kvb, kv, mask, Dn, Dr, Dv, Dl, scale)
    return dense, expected, dict(q=q_dense, kvb=kvb, kv=kv, mask=mask, idx=idx, cnt=cnt)


def pin_dense_equals_absorbed_then_up_projected():
    """With the no-rope keys and the values up-projected from the latent
    rows (k = Wkb c, v = Wvb c) and the absorbed query Wkb^T q_nope, the
    dense masked form equals the absorbed sparse attention (itself pinned)
    followed by the value up-projection, in exact arithmetic.  Positions
    span both regimes: fewer causal keys than top_k (every earlier key) and
    a real top-k selection."""
    rng = np.random.default_rng(21)
    dense, expected, _ = _dense_absorbed_pair(rng, L=24, N=30, H=3, Dl=64, Dn=48, Dr=16, Dv=40,
                                              q_start=4, top_k=16, scale=1 / 8)
    assert np.abs(expected).max() > 1
    assert np.allclose(dense, expected, rtol=1e-11, atol=1e-11 * np.abs(expected).max())


def pin_selection_mask_brute_force():
    """The mask holds exactly the selected keys that are in range and
    causal: padding (-1), ids at or past N, keys after the query's position
    and entries past count are left out; count is clamped to [0, top_k]."""
    idx = np.array([[0, 3, 5, -1], [2, 9, 40, 1], [7, 6, 33, 64], [1, 2, 3, 4], [0, 1, 2, 3]], np.int32)
    cnt = np.array([3, 4, 4, -2, 9], np.int32)
    q_start, N = 5, 40
    mask = oracle.selection_mask(idx, cnt, N, q_start)
    assert mask.shape == (5, 2)
    for i in range(5):
        want = set()
        for t in range(max(0, min(int(cnt[i]), 4))):
            j = int(idx[i, t])
            if 0 <= j < N and j <= q_start + i:
                want.add(j)
        got = {32 * w + b for w in range(mask.shape[1]) for b in range(32) if (int(mask[i, w]) >> b) & 1}
        assert got == want, (i, got, want)
    assert oracle.selection_mask(idx, cnt, N, q_start, W=3).shape == (5, 3)


def pin_dense_closed_forms():
    """One masked-in key returns that key's value exactly; no masked-in key
    returns zeros; two keys whose scores differ by d split their weight as
    1 : e^(scale d), through the rope part alone."""
    rng = np.random.default_rng(22)
    L, N, H, Dn, Dr, Dv = 3, 6, 2, 32, 16, 24
    q = _bf(rng.standard_normal((L, H, Dn + Dr)).astype(np.float32))
    kvb = _bf(rng.standard_normal((N, H, Dn + Dv)).astype(np.float32))
    kv = _bf(rng.standard_normal((N, 8 + Dr)).astype(np.float32))
    mask = np.zeros((L, 2), np.uint32)
    mask[0, 0] = 1 << 4          # key 4 only
    mask[2, 0] = (1 << 1) | (1 << 5)
    out = oracle.dense_masked_attn(q, kvb, kv, mask, Dn, Dr, Dv, 8, 0.125)
    assert np.array_equal(out[0], _f(kvb[4, :, Dn:]))
    assert np.array_equal(out[1], np.zeros((H, Dv)))
    # keys 1 and 5 with equal no-rope keys; the rope keys differ in one column
    q2 = np.zeros((L, H, Dn + Dr), np.float32)
    q2[2, :, Dn + 3] = 2.0
    kvb2 = _f(kvb).astype(np.float32)
    kvb2[5, :, :Dn] = kvb2[1, :, :Dn]
    kv2 = np.zeros((N, 8 + Dr), np.float32)
    kv2[1, 8 + 3], kv2[5, 8 + 3] = 1.5, -0.5
    out = oracle.dense_masked_attn(_bf(q2), _bf(kvb2), _bf(kv2), mask, Dn, Dr, Dv, 8, 0.125)
    w1 = 1.0 / (1.0 + math.exp(0.125 * 2.0 * (-0.5 - 1.5)))
    want = w1 * kvb2[1, :, Dn:].astype(np.float64) + (1 - w1) * kvb2[5, :, Dn:].astype(np.float64)
    assert np.allclose(out[2], want, rtol=1e-12, atol=1e-12)


def _f16_bits_to_f64(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def pin_kv_b_f16_rounding_closed_forms():
    """One-hot weights copy a latent value: bf16 keys unchanged, values as
    numpy's float16 of it; sums that land between fp16 neighbours round to
    nearest with ties to even (1 + 2^-11 -> 1, 1 + 3*2^-11 -> 1 + 2^-9,
    65504 + 16 -> inf, 2^-25 + 2^-26 -> the smallest subnormal 2^-24)."""
    N, H, Dl, Dn, Dv = 3, 2, 64, 8, 8
    rng = np.random.default_rng(31)
    kv = _bf(rng.standard_normal((N, Dl + 16)).astype(np.float32))
    w = np.zeros((H * (Dn + Dv), Dl), np.uint16)
    cols = rng.integers(0, Dl, size=H * (Dn + Dv))
    w[np.arange(H * (Dn + Dv)), cols] = 0x3F80
    for f16 in (False, True):
        out = oracle.kv_b_proj(kv, w, H, Dl, Dn, Dv, f16).reshape(N, H * (Dn + Dv))
        lat = kv[:, cols].reshape(N, H, Dn + Dv)
        got = out.reshape(N, H, Dn + Dv)
        assert np.array_equal(got[..., :Dn], lat[..., :Dn])
        want_v = W.bf16_bits_to_f32(lat[..., Dn:]).astype(np.float16).view(np.uint16) if f16 else lat[..., Dn:]
        assert np.array_equal(got[..., Dn:], want_v)
    # two-term sums around fp16 rounding points (value column 0 of head 0)
    cases = [(1.0, 2.0 ** -11, 1.0), (1.0, 3 * 2.0 ** -11, 1.0 + 2.0 ** -9), (65504.0, 16.0, np.inf),
             (2.0 ** -25, 2.0 ** -26, 2.0 ** -24), (-1.0, -(2.0 ** -11), -1.0)]
    for a, b, want in cases:
        kv2 = np.zeros((1, Dl), np.uint16)
        kv2[0, 0], kv2[0, 1] = _bf(np.float32(a)), _bf(np.float32(b))
        w2 = np.zeros((Dn + Dv, Dl), np.uint16)
        w2[Dn, 0] = w2[Dn, 1] = 0x3F80
        got = _f16_bits_to_f64(oracle.kv_b_proj(kv2, w2, 1, Dl, Dn, Dv, True)[0, 0, Dn])
        assert got == want, (a, b, got, want)


def pin_kv_b_matches_numpy():
    """Random bf16 latent rows and weights: every output within half a unit
    of its format (bf16 keys, fp16 or bf16 values) of numpy's float64
    product; integer data gives the exact sums."""
    rng = np.random.default_rng(32)
    N, H, Dl, Dn, Dv, kc = 7, 3, 64, 16, 24, 80
    kv = _bf(rng.standard_normal((N, kc)).astype(np.float32))
    w = _bf((rng.standard_normal((H * (Dn + Dv), Dl)) / 8).astype(np.float32))
    ref = (_f(kv)[:, :Dl] @ _f(w).T).reshape(N, H, Dn + Dv)
    for f16 in (False, True):
        got = oracle.kv_b_proj(kv, w, H, Dl, Dn, Dv, f16)
        k = _f(got[..., :Dn])
        assert np.all(np.abs(k - ref[..., :Dn]) <= _half_ulp_bf16(ref[..., :Dn]) * 1.0000001 + 1e-30)
        if f16:
            v = _f16_bits_to_f64(got[..., Dn:])
            r = ref[..., Dn:]
            ulp = np.spacing(np.abs(r).astype(np.float16)).astype(np.float64)
            assert np.all(np.abs(v - r) <= ulp / 2 * 1.0000001 + 2.0 ** -25)
        else:
            assert np.all(np.abs(_f(got[..., Dn:]) - ref[..., Dn:]) <= _half_ulp_bf16(ref[..., Dn:]) * 1.0000001 + 1e-30)
    lat = rng.integers(-2, 3, size=(N, Dl))
    wi = rng.integers(-1, 2, size=(H * (Dn + Dv), Dl))
    got = oracle.kv_b_proj(_bf(lat), _bf(wi), H, Dl, Dn, Dv, True)
    exact = (lat @ wi.T).reshape(N, H, Dn + Dv)
    assert np.array_equal(_f(got[..., :Dn]), exact[..., :Dn])
    assert np.array_equal(_f16_bits_to_f64(got[..., Dn:]), exact[..., Dn:])


def pin_q_absorb_one_hot():
    """Key rows of the kv_b weight that copy no-rope query column c to latent
    column perm[c]: the absorbed query holds q[..., c] at perm[c] exactly and
    zero elsewhere, whatever the value rows hold; the rope part is copied."""
    T, H, Dn, Dr, Dl, Dv = 3, 2, 8, 4, 32, 8
    rng = np.random.default_rng(41)
    q = _bf(rng.standard_normal((T, H, Dn + Dr)).astype(np.float32))
    w = _bf(rng.standard_normal((H * (Dn + Dv), Dl)).astype(np.float32))   # value rows: noise
    perm = np.stack([rng.permutation(Dl)[:Dn] for _ in range(H)])
    for h in range(H):
        w[h * (Dn + Dv):h * (Dn + Dv) + Dn] = 0
        w[h * (Dn + Dv) + np.arange(Dn), perm[h]] = 0x3F80
    out = oracle.q_absorb(q, w, Dl, Dn, Dv)
    assert out.shape == (T, H, Dl + Dr)
    for h in range(H):
        want = np.zeros((T, Dl), np.uint16)
        want[:, perm[h]] = q[:, h, :Dn]
        assert np.array_equal(out[:, h, :Dl], want)
    assert np.array_equal(out[..., Dl:], q[..., Dn:])


def pin_q_absorb_score_invariant():
    """The absorbed query scores a latent row as the no-rope query scores
    that row's up-projected key: <absorb(q), kv> = <q, W_UK kv>, up to the
    bf16 rounding of the absorbed query (half a unit per element).  Against
    numpy's float64 products, with integer data exactly."""
    T, H, Dn, Dr, Dl, Dv, N = 4, 3, 16, 8, 64, 24, 5
    rng = np.random.default_rng(42)
    q = _bf(rng.standard_normal((T, H, Dn + Dr)).astype(np.float32))
    w = _bf((rng.standard_normal((H * (Dn + Dv), Dl)) / 8).astype(np.float32))
    kv = _f(_bf(rng.standard_normal((N, Dl)).astype(np.float32)))
    out = _f(oracle.q_absorb(q, w, Dl, Dn, Dv)[..., :Dl])
    wk = _f(w).reshape(H, Dn + Dv, Dl)[:, :Dn]                 # [H, Dn, Dl]
    exact = np.einsum("thc,hcd->thd", _f(q[..., :Dn]), wk)     # float64
    assert np.all(np.abs(out - exact) <= _half_ulp_bf16(exact) * 1.0000001 + 1e-30)
    kvb_key = np.einsum("hcd,nd->nhc", wk, kv)                 # the up-projected keys
    lhs = np.einsum("thd,nd->thn", out, kv)
    rhs = np.einsum("thc,nhc->thn", _f(q[..., :Dn]), kvb_key)
    bound = np.einsum("thd,nd->thn", np.abs(out), np.abs(kv)) * 2.0 ** -8
    assert np.all(np.abs(lhs - rhs) <= bound + 1e-12)
    qi = rng.integers(-2, 3, size=(T, H, Dn + Dr))
    wi = rng.integers(-1, 2, size=(H * (Dn + Dv), Dl))
    got = _f(oracle.q_absorb(_bf(qi), _bf(wi), Dl, Dn, Dv))
    ex = np.einsum("thc,hcd->thd", qi[..., :Dn], wi.reshape(H, Dn + Dv, Dl)[:, :Dn])
    assert np.array_equal(got[..., :Dl], ex) and np.array_equal(got[..., Dl:], qi[..., Dn:])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
