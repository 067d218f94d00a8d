"""GPU parity of the projections (dsa_value_up_proj, dsa_o_proj, and the
dense path's dsa_kv_b_proj) against the CPU oracle on the same seeded inputs.

Tolerances, from the arithmetic:
- up-projection: both sides round the float32 attention output to bf16 and
  the result once to bf16; they differ only in the summation (fp32 on the
  GPU, exact on the CPU).  An output may therefore land one bf16 unit away
  where the exact sum lies next to a rounding midpoint, and where the sum
  cancels to far below its terms the fp32 summation error (a few 2^-24 of
  the sum of |terms|) can exceed a bf16 unit of the small result.  Bound:
  |g - r| <= 1 bf16 unit of r + 2^-20 * sum |terms|, and under 1% of the
  outputs differ at all;
- output projection: same bf16 operands, fp32 against exact accumulation
  over k_in terms: max |y - r| / max |r| per row <= 1e-5.
Cases: the 16k chunk's 4096 tokens (the launch the benchmark times; the
oracle runs on a seeded sample of rows), 8 decode tokens, and 37 tokens (a
partial row tile)."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import dev, host, requires_gpu, row_rel_err, say, vt_position

pytestmark = [pytest.mark.gpu, requires_gpu]


def rows_of(cfg):
    return np.arange(cfg.T) if cfg.T <= 64 else W.sample_rows(cfg.T, 24, seed=5)


def ulp_distance(a, b):
    """Distance in bf16 units between bit patterns (same-sign ordering)."""
    def key(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x & 0x7FFF)
    return np.abs(key(a) - key(b))


def run_up(cfg, d):
    import torch
    import sparse_attention_scores_amd as dsa
    out = torch.empty((cfg.T, cfg.H, cfg.Dv), dtype=torch.int16, device="cuda")
    dsa.dsa_value_up_proj(W.GLM, dev(d["o"]), dev(d["wv"]), cfg.T, cfg.Dv, out)
    return host(out)


def run_oproj(cfg, x):
    import torch
    import sparse_attention_scores_amd as dsa
    y = torch.empty((cfg.T, cfg.hidden), dtype=torch.float32, device="cuda")
    dsa.dsa_o_proj(dev(x), dev(d_wo(cfg)), cfg.T, cfg.H * cfg.Dv, cfg.hidden, y)
    return host(y)


_cache = {}


def inputs(name):
    if name not in _cache:
        _cache.clear()
        _cache[name] = W.make_proj(W.PROJ[name])
    return _cache[name]


def d_wo(cfg):
    return inputs(cfg.name)["wo"]


@pytest.mark.parametrize("name", list(W.PROJ))
def test_value_up_proj_matches_oracle(name):
    cfg = W.PROJ[name]
    d = inputs(name)
    say("value_up_proj", name, "T=%d" % cfg.T)
    got = run_up(cfg, d)
    rows = rows_of(cfg)
    want = oracle.value_up_proj(d["o"][rows], d["wv"])
    dist = ulp_distance(got[rows], want)
    assert (dist > 0).mean() < 0.01, float((dist > 0).mean())
    g = W.bf16_bits_to_f32(got[rows]).astype(np.float64)
    r = W.bf16_bits_to_f32(want).astype(np.float64)
    ob = np.abs(W.bf16_bits_to_f32(W.to_bf16_bits(d["o"][rows])).astype(np.float64))
    wa = np.abs(W.bf16_bits_to_f32(d["wv"]).astype(np.float64))
    terms = np.einsum("thc,hjc->thj", ob, wa)
    unit = np.ldexp(1.0, (np.floor(np.log2(np.maximum(np.abs(r), 1e-38))) - 7).astype(int))
    excess = np.abs(g - r) - (unit + 2.0 ** -20 * terms)
    assert excess.max() <= 0, float(excess.max())


@pytest.mark.parametrize("name", list(W.PROJ))
def test_o_proj_matches_oracle(name):
    cfg = W.PROJ[name]
    d = inputs(name)
    say("o_proj", name, "T=%d" % cfg.T)
    y = run_oproj(cfg, d["x"])
    rows = rows_of(cfg)
    ref = oracle.o_proj(d["x"], d["wo"], rows)
    err = row_rel_err(y[rows], ref)
    assert err <= 1e-5, err


def test_projections_end_to_end():
    """up-projection output fed to the output projection, against the oracle
    doing both steps (its own bf16 out_v): a one-unit difference in a few
    out_v values moves y by far less than 1e-3 of the row."""
    cfg = W.PROJ["glm_small"]
    d = inputs("glm_small")
    say("projections end to end", cfg.name)
    out_v = run_up(cfg, d)
    y = run_oproj(cfg, out_v.reshape(cfg.T, cfg.H * cfg.Dv))
    ov = oracle.value_up_proj(d["o"], d["wv"])
    ref = oracle.o_proj(ov.reshape(cfg.T, cfg.H * cfg.Dv), d["wo"])
    err = row_rel_err(y, ref)
    assert err <= 1e-3, err


# ---------------------------------------------------------------- kv_b (dense path)
def _values(bits, f16):
    b = np.asarray(bits, dtype=np.uint16)
    return (b.view(np.float16) if f16 else W.bf16_bits_to_f32(b)).astype(np.float64)


@pytest.mark.parametrize("name,f16", [("glm_8k_chunk", True), ("glm_small", True), ("glm_small", False),
                                      ("tiny", True)])
def test_kv_b_proj_matches_oracle(name, f16):
    """bf16 keys and fp16 (or bf16) values of the kv_b product, against the
    oracle's exactly summed, once-rounded results: both sides take the same
    bf16 operands and round once; they differ in the summation (fp32 against
    exact).  Bound per output: one unit of its format + 2^-20 * sum |terms|,
    and under 1% of outputs differ at all.  glm_8k_chunk: 8192 keys (the
    benchmark's launch), on a seeded sample of 48 rows; glm_small: 700 keys
    (a partial row tile); tiny: 4 heads x (64 + 64)."""
    import torch
    import sparse_attention_scores_amd as dsa
    cfg = W.DENSE[name]
    d = W.make_dense(cfg)
    w = W.make_kvb_weight(cfg)
    C = cfg.Dn + cfg.Dv
    kc = cfg.Dl + cfg.Dr
    say("kv_b_proj", name, "N=%d" % cfg.N, "f16" if f16 else "bf16")
    out = torch.zeros((cfg.N, cfg.H, C), dtype=torch.int16, device="cuda")
    Np = dsa.vt_keys(cfg.N)
    vt = torch.full((cfg.H, cfg.Dv, Np), -1, dtype=torch.int16, device="cuda") if f16 else None
    dsa.dsa_kv_b_proj(dev(d["kv"]), kc, dev(w), cfg.N, cfg.H, cfg.Dl, cfg.Dn, cfg.Dv, out, vt)
    got = host(out)
    if f16:
        # values from the vt form back to [N, H, Dv]; its padding must be zeros
        vh = host(vt)
        pos = vt_position(np.arange(cfg.N))
        assert not vh[:, :, np.setdiff1d(np.arange(Np), pos)].any()
        got[..., cfg.Dn:] = np.transpose(vh[:, :, pos], (2, 0, 1))
    rows = np.arange(cfg.N) if cfg.N <= 1024 else W.sample_rows(cfg.N, 48, seed=11, must=[0, cfg.N - 1])
    want = oracle.kv_b_proj(d["kv"][rows], w, cfg.H, cfg.Dl, cfg.Dn, cfg.Dv, f16)
    g = got[rows]
    assert (g != want).mean() < 0.01, float((g != want).mean())
    lat = np.abs(W.bf16_bits_to_f32(d["kv"][rows, :cfg.Dl]).astype(np.float64))
    terms = (lat @ np.abs(W.bf16_bits_to_f32(w).astype(np.float64)).T).reshape(len(rows), cfg.H, C)
    for sl, is16, mant in ((np.s_[..., :cfg.Dn], False, 7), (np.s_[..., cfg.Dn:], f16, 10 if f16 else 7)):
        gv, rv = _values(g[sl], is16), _values(want[sl], is16)
        assert np.isfinite(gv).all()
        unit = np.ldexp(1.0, (np.floor(np.log2(np.maximum(np.abs(rv), 2.0 ** -14))) - mant).astype(int))
        excess = np.abs(gv - rv) - (unit + 2.0 ** -20 * terms[sl])
        assert excess.max() <= 0, float(excess.max())


# ---------------------------------------------------------------- query absorption
@pytest.mark.parametrize("name", ["glm_8k_chunk", "glm_small"])
def test_q_absorb_matches_oracle(name):
    """The absorbed query (no-rope query times each head's key block of the
    kv_b weight, rope part copied) against the oracle, which sums exactly from
    the untransposed weight and rounds once.  dsa_absorb_weight's transposed
    key block must equal numpy's transpose bit for bit; the rope columns are
    copies.  Latent columns: same bf16 operands, fp32 against exact sums, so
    one bf16 unit + 2^-20 * sum |terms| per output, under 1% of outputs
    differing.  glm_8k_chunk: 4096 tokens (the benchmark's launch) on a
    seeded sample of 24 rows; glm_small: 160 tokens (a partial row tile)."""
    import torch
    import sparse_attention_scores_amd as dsa
    cfg = W.DENSE[name]
    d = W.make_dense(cfg)
    w = W.make_kvb_weight(cfg)
    H, Dn, Dr, Dl, Dv = cfg.H, cfg.Dn, cfg.Dr, cfg.Dl, cfg.Dv
    say("q_absorb", name, "T=%d" % cfg.L)
    wk_t = torch.empty((H, Dl, Dn), dtype=torch.int16, device="cuda")
    dsa.dsa_absorb_weight(dev(w), H, Dn, Dv, Dl, wk_t)
    want_t = np.ascontiguousarray(np.transpose(w.reshape(H, Dn + Dv, Dl)[:, :Dn], (0, 2, 1)))
    assert np.array_equal(host(wk_t).view(np.uint16), want_t)
    q_abs = torch.full((cfg.L, H, Dl + Dr), -1, dtype=torch.int16, device="cuda")
    dsa.dsa_q_absorb(dev(d["q"]), wk_t, cfg.L, H, Dn, Dr, Dl, q_abs)
    got = host(q_abs).view(np.uint16)
    rows = np.arange(cfg.L) if cfg.L <= 256 else W.sample_rows(cfg.L, 24, seed=13, must=[0, cfg.L - 1])
    want = oracle.q_absorb(d["q"][rows], w, Dl, Dn, Dv)
    g = got[rows]
    assert np.array_equal(g[..., Dl:], want[..., Dl:])
    gl, rl = g[..., :Dl], want[..., :Dl]
    assert (gl != rl).mean() < 0.01, float((gl != rl).mean())
    qa = np.abs(W.bf16_bits_to_f32(d["q"][rows, :, :Dn]).astype(np.float64))
    wa = np.abs(W.bf16_bits_to_f32(want_t).astype(np.float64))
    terms = np.einsum("thc,hdc->thd", qa, wa)
    gv = W.bf16_bits_to_f32(gl).astype(np.float64)
    rv = W.bf16_bits_to_f32(rl).astype(np.float64)
    unit = np.ldexp(1.0, (np.floor(np.log2(np.maximum(np.abs(rv), 1e-38))) - 7).astype(int))
    excess = np.abs(gv - rv) - (unit + 2.0 ** -20 * terms)
    assert excess.max() <= 0, float(excess.max())


def test_q_absorb_rejects_unsupported_shapes():
    import torch
    import sparse_attention_scores_amd as dsa
    q = torch.zeros((4, 2, 128), dtype=torch.int16, device="cuda")
    wk_t = torch.zeros((2, 256, 64), dtype=torch.int16, device="cuda")
    out = torch.zeros((4, 2, 320), dtype=torch.int16, device="cuda")
    with pytest.raises(dsa.DsaError):
        dsa.dsa_q_absorb(q, wk_t, 4, 2, 48, 80, 256, out)    # d_nope not a multiple of 64
    with pytest.raises(dsa.DsaError):
        dsa.dsa_q_absorb(q, wk_t, 4, 2, 64, 64, 192, out)    # d_latent not a multiple of 256
