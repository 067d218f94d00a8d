"""Seeded synthetic inputs for the DSA prefill/decode path.

This module only draws random numbers and rounds them to bf16 storage.  It
holds none of the method's arithmetic, so both the CPU oracle's tests and the
GPU path take their inputs from here without sharing any computation.

Shapes follow the GLM-5.x ``glm_moe_dsa`` configuration printed in the text
config of "GLM-5.2-Vision: llama.cpp vs vLLM line-by-line pipeline trace"
(64 heads, kv_lora_rank 512, qk_rope 64, index_topk 2048) and the indexer
description in exo PR #2539 (Prefill section, float32 indexer item: 32
indexer heads).  The indexer width 128 is not on the pages; it is the
DeepSeek-V3.2 indexer head size and is taken as a parameter.

Value recipe:
  draw order  qI, kI, w, q, kv from ``numpy.random.default_rng(seed)``;
  qI, kI      integers uniform in [-r, r] (r = 4 tiny, 8 GLM), exact in bf16;
  w           uniform choice of {0.5, 1, 2} (powers of two), fp32;
  q, kv       standard normal (float32) times a scale, rounded once to bf16
              (round to nearest even).

With integer indexer operands and power-of-two weights every partial sum of
the indexer is a multiple of 0.5 below 2**20, so fp32 accumulation in any
order is exact; selection can then be compared bit for bit.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "Shape", "TINY", "GLM", "Prefill", "Decode", "PREFILL", "DECODE",
    "to_bf16_bits", "bf16_bits_to_f32", "make_prefill", "make_prefill_fp16_range", "make_decode",
    "CacheWrite", "CACHE_WRITE", "make_cache_write", "Router", "ROUTER", "make_router",
    "Proj", "PROJ", "make_proj",
]


@dataclasses.dataclass(frozen=True)
class Shape:
    n_heads: int          # H   query heads
    d_latent: int         # Dl  absorbed no-rope width == value width
    d_rope: int           # Dr  rope width
    n_idx_heads: int      # Hi  indexer heads
    d_idx: int            # Di  indexer head width
    top_k: int            # keys kept per query
    softmax_scale: float = 1.0 / 16.0

    @property
    def d_qk(self) -> int:
        return self.d_latent + self.d_rope


# GLM-5.x glm_moe_dsa layer (pipeline-trace config line; exo #2539 indexer).
GLM = Shape(n_heads=64, d_latent=512, d_rope=64, n_idx_heads=32, d_idx=128, top_k=2048)
# Tiny check shape: 4 heads, latent 64 + rope 16, indexer 4 x 32, top_k 32.
TINY = Shape(n_heads=4, d_latent=64, d_rope=16, n_idx_heads=4, d_idx=32, top_k=32)


@dataclasses.dataclass(frozen=True)
class Prefill:
    name: str
    shape: Shape
    L: int                # queries in the chunk
    q_start: int          # position of the first query
    seed: int
    int_range: int        # indexer integers in [-int_range, int_range]
    q_scale: float
    kv_scale: float

    @property
    def N(self) -> int:   # keys: every position up to the chunk's last query
        return self.q_start + self.L


@dataclasses.dataclass(frozen=True)
class Decode:
    name: str
    shape: Shape
    ctx: tuple            # context length per sequence; query at ctx-1
    seed: int
    int_range: int
    q_scale: float
    kv_scale: float


PREFILL: Dict[str, Prefill] = {
    # tiny fp32-generated check: L=64 at 192..255 over 256 keys, top_k 32
    "tiny": Prefill("tiny", TINY, 64, 192, 0, 4, 1.0, 1.0),
    # tiny shape with top_k 256: every query takes the every-earlier-key rule
    "tiny_dense": Prefill("tiny_dense", dataclasses.replace(TINY, top_k=256), 64, 192, 10, 4, 1.0, 1.0),
    # tiny shape with a peaked softmax (queries scaled by 4)
    "tiny_sharp": Prefill("tiny_sharp", TINY, 64, 192, 11, 4, 4.0, 1.0),
    # GLM-shape chunk, 4096 queries at 4096..8191 over 8192 keys
    "glm_8k": Prefill("glm_8k", GLM, 4096, 4096, 1, 8, 0.05, 0.05),
    # first chunk: queries 0..4095; those below 2048 take every earlier key
    "glm_first_4k": Prefill("glm_first_4k", GLM, 4096, 0, 2, 8, 0.05, 0.05),
    # long-context chunk, 4096 queries at 12288..16383 over 16384 keys
    "glm_16k": Prefill("glm_16k", GLM, 4096, 12288, 3, 8, 0.05, 0.05),
    # small GLM-shape chunks the oracle finishes quickly; ragged sizes that
    # span several tiles and cross the top_k boundary inside the chunk
    "glm_small_cross": Prefill("glm_small_cross", GLM, 77, 2011, 21, 8, 0.05, 0.05),
    "glm_small_sparse": Prefill("glm_small_sparse", GLM, 45, 3001, 22, 8, 0.05, 0.05),
    "glm_small_first": Prefill("glm_small_first", GLM, 33, 0, 23, 8, 0.05, 0.05),
}

DECODE: Dict[str, Decode] = {
    # batched decode: 8 sequences, contexts 4k..64k
    "glm_decode_8": Decode("glm_decode_8", GLM,
                           (4096, 8192, 16384, 32768, 65536, 65536, 16384, 4096), 4, 8, 0.05, 0.05),
    # small ragged decode the oracle finishes quickly (one context below top_k)
    "glm_decode_small": Decode("glm_decode_small", GLM, (3000, 1500, 2049, 2048, 4133), 24, 8, 0.05, 0.05),
    "tiny_decode": Decode("tiny_decode", TINY, (256, 31, 100, 1, 33), 25, 4, 1.0, 1.0),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.
    uint32 arithmetic cannot overflow for finite inputs (the largest finite
    pattern plus 0x8000 stays below 2**32)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng: np.random.Generator, shape: Shape, n_q: int, n_k: int, r: int,
          q_scale: float, kv_scale: float) -> Dict[str, np.ndarray]:
    """Draw one set of operands in the fixed order qI, kI, w, q, kv."""
    qI = rng.integers(-r, r + 1, size=(n_q, shape.n_idx_heads, shape.d_idx)).astype(np.float32)
    kI = rng.integers(-r, r + 1, size=(n_k, shape.d_idx)).astype(np.float32)
    w = rng.choice(np.array([0.5, 1.0, 2.0], dtype=np.float32), size=(n_q, shape.n_idx_heads))
    q = rng.standard_normal(size=(n_q, shape.n_heads, shape.d_qk), dtype=np.float32) * np.float32(q_scale)
    kv = rng.standard_normal(size=(n_k, shape.d_qk), dtype=np.float32) * np.float32(kv_scale)
    return {
        "qI": to_bf16_bits(qI), "kI": to_bf16_bits(kI), "w": np.ascontiguousarray(w, dtype=np.float32),
        "q": to_bf16_bits(q), "kv": to_bf16_bits(kv),
    }


def make_prefill(cfg: Prefill) -> Dict[str, np.ndarray]:
    """Inputs of one prefill chunk.  Keys sit at positions 0..N-1."""
    rng = np.random.default_rng(cfg.seed)
    return _draw(rng, cfg.shape, cfg.L, cfg.N, cfg.int_range, cfg.q_scale, cfg.kv_scale)


def make_prefill_fp16_range(cfg: Prefill) -> Dict[str, np.ndarray]:
    """Inputs of one prefill chunk whose attention operands span the fp16
    range: the indexer operands as make_prefill draws them, then (from a
    second generator seeded cfg.seed + 1000) q and kv with a log-uniform
    magnitude per element, rounded to bf16.
      kv latent   N(0,1) * 2**U(-27, 15), clipped to +-2**15 (a third of the
                  values below fp16's normal range 2**-14, the largest 2**15);
      kv rope     N(0,1) * 2**U(-6, 2);
      q latent    N(0,1) * 2**U(-30, -9) (most values fp16 subnormals);
      q rope      N(0,1) * 2**U(-8, -3).
    The softmax stays spread (the largest probability of a row is typically
    about 0.3)."""
    d = make_prefill(cfg)
    rng = np.random.default_rng(cfg.seed + 1000)
    sh = cfg.shape

    def wide(shape, lo, hi, cap=None):
        x = rng.standard_normal(size=shape) * 2.0 ** rng.uniform(lo, hi, size=shape)
        if cap is not None:
            x = np.clip(x, -cap, cap)
        return x.astype(np.float32)

    kv = np.concatenate([wide((cfg.N, sh.d_latent), -27, 15, 2.0 ** 15), wide((cfg.N, sh.d_rope), -6, 2)], axis=1)
    q = np.concatenate([wide((cfg.L, sh.n_heads, sh.d_latent), -30, -9),
                        wide((cfg.L, sh.n_heads, sh.d_rope), -8, -3)], axis=2)
    d["q"], d["kv"] = to_bf16_bits(q), to_bf16_bits(kv)
    return d


def make_decode(cfg: Decode) -> Dict[str, np.ndarray]:
    """Inputs of one batched decode step: one query per sequence, caches packed
    in sequence order (rows of sequence b start at sum(ctx[:b]))."""
    rng = np.random.default_rng(cfg.seed)
    d = _draw(rng, cfg.shape, len(cfg.ctx), int(sum(cfg.ctx)), cfg.int_range, cfg.q_scale, cfg.kv_scale)
    d["ctx"] = np.asarray(cfg.ctx, dtype=np.int64)
    d["row_off"] = np.concatenate([[0], np.cumsum(d["ctx"])]).astype(np.int64)
    return d


def sample_rows(L: int, n: int, seed: int = 1234, must: Optional[List[int]] = None) -> np.ndarray:
    """A sorted, seeded sample of n query rows out of L, always holding the
    first and last row and any rows listed in ``must``."""
    rng = np.random.default_rng(seed)
    pick = set(int(x) for x in rng.choice(L, size=min(n, L), replace=False))
    pick.update([0, L - 1])
    for m in must or []:
        if 0 <= m < L:
            pick.add(int(m))
    return np.array(sorted(pick), dtype=np.int64)


@dataclasses.dataclass(frozen=True)
class CacheWrite:
    """T new tokens written into caches of N rows (the upstream cache write).
    ``positions``: "chunk" = p0 .. p0+T-1; "scatter" = T distinct seeded
    positions in [0, N) that include 0 and N-1, plus (if ``bad``) one
    position -1 and one position N, whose cache rows must not be written."""
    name: str
    shape: Shape
    T: int
    N: int
    p0: int
    positions: str
    seed: int
    bad: bool = False
    d_idx_rope: int = 64
    theta: float = 10000.0
    eps: float = 1e-6


CACHE_WRITE: Dict[str, CacheWrite] = {
    # the 16k chunk's 4096 new tokens at positions 12288..16383
    "glm_16k_chunk": CacheWrite("glm_16k_chunk", GLM, 4096, 16384, 12288, "chunk", 31),
    # eight decode tokens scattered over a 64k-row cache
    "glm_decode_8": CacheWrite("glm_decode_8", GLM, 8, 65536, 0, "scatter", 32),
    # small ragged cases the oracle finishes at once
    "glm_small": CacheWrite("glm_small", GLM, 37, 300, 0, "scatter", 33, bad=True),
    "tiny": CacheWrite("tiny", TINY, 29, 64, 0, "scatter", 34, bad=True, d_idx_rope=16),
}


def make_cache_write(cfg: CacheWrite) -> Dict[str, np.ndarray]:
    """Inputs of one cache write, drawn in the order positions, kv_a, norm_w,
    kI_new, q, qI, kv_cache, kI_cache.  kv_a, q and the indexer rows are
    standard normal rounded to bf16; the norm weight is 1 + 0.1 N(0,1) in
    fp32; the caches start as standard normal rows (so rows that must stay
    untouched are visible)."""
    sh = cfg.shape
    rng = np.random.default_rng(cfg.seed)
    if cfg.positions == "chunk":
        pos = np.arange(cfg.p0, cfg.p0 + cfg.T, dtype=np.int64)
    else:
        n_good = cfg.T - (2 if cfg.bad else 0)
        pick = rng.choice(np.arange(1, cfg.N - 1), size=n_good - 2, replace=False)
        pos = np.concatenate([[0, cfg.N - 1], pick] + ([[-1, cfg.N]] if cfg.bad else []))
        pos = rng.permutation(pos).astype(np.int64)
    nrm = lambda *shp: rng.standard_normal(size=shp, dtype=np.float32)
    kv_a = to_bf16_bits(nrm(cfg.T, sh.d_qk))
    norm_w = (np.float32(1.0) + np.float32(0.1) * nrm(sh.d_latent)).astype(np.float32)
    kI_new = to_bf16_bits(nrm(cfg.T, sh.d_idx))
    q = to_bf16_bits(nrm(cfg.T, sh.n_heads, sh.d_qk))
    qI = to_bf16_bits(nrm(cfg.T, sh.n_idx_heads, sh.d_idx))
    kv_cache = to_bf16_bits(nrm(cfg.N, sh.d_qk))
    kI_cache = to_bf16_bits(nrm(cfg.N, sh.d_idx))
    return {"pos": pos, "kv_a": kv_a, "norm_w": norm_w, "kI_new": kI_new, "q": q, "qI": qI,
            "kv_cache": kv_cache, "kI_cache": kI_cache}


@dataclasses.dataclass(frozen=True)
class Router:
    """Router selection over T tokens: E experts, k kept per token, scaled by
    ``scale`` (GLM: 256 experts, 8 per token, routed_scaling_factor 2.5).
    ``kind``: "normal" = logits N(0,1)*2 and bias N(0,1)*0.1; "ties" =
    integer logits in [-1, 1] and a bias of 0 or +-2^-10 (many exactly equal
    selection scores); "tiny_p" = logits near -30 (probabilities far below
    the weight-sum clamp)."""
    name: str
    T: int
    E: int
    k: int
    seed: int
    kind: str = "normal"
    scale: float = 2.5


ROUTER: Dict[str, Router] = {
    "glm_16k_chunk": Router("glm_16k_chunk", 4096, 256, 8, 41),
    "glm_decode_8": Router("glm_decode_8", 8, 256, 8, 42),
    "glm_ties": Router("glm_ties", 64, 256, 8, 43, "ties"),
    "glm_tiny_p": Router("glm_tiny_p", 16, 256, 8, 44, "tiny_p"),
    "small": Router("small", 33, 64, 4, 45),
    "small_ties": Router("small_ties", 40, 128, 6, 46, "ties"),
}


def make_router(cfg: Router) -> Dict[str, np.ndarray]:
    """Router logits [T, E] and bias [E], float32, drawn in that order."""
    rng = np.random.default_rng(cfg.seed)
    if cfg.kind == "ties":
        logits = rng.integers(-1, 2, size=(cfg.T, cfg.E)).astype(np.float32)
        bias = (rng.integers(-1, 2, size=cfg.E) * 2.0 ** -10).astype(np.float32)
    elif cfg.kind == "tiny_p":
        logits = (-30.0 + rng.standard_normal(size=(cfg.T, cfg.E))).astype(np.float32)
        bias = (rng.standard_normal(size=cfg.E) * 0.1).astype(np.float32)
    else:
        logits = (rng.standard_normal(size=(cfg.T, cfg.E)) * 2.0).astype(np.float32)
        bias = (rng.standard_normal(size=cfg.E) * 0.1).astype(np.float32)
    return {"logits": np.ascontiguousarray(logits), "bias": np.ascontiguousarray(bias)}


@dataclasses.dataclass(frozen=True)
class Proj:
    """Downstream projections of T tokens: the attention output o [T, H, Dl]
    (float32) goes through the per-head value up-projection wv [H, Dv, Dl]
    and the output projection wo [hidden, H*Dv] (GLM: 64 heads, Dl 512,
    v_head_dim 256, hidden 6144 from the pipeline trace's config line)."""
    name: str
    T: int
    seed: int
    H: int = 64
    Dl: int = 512
    Dv: int = 256
    hidden: int = 6144


PROJ: Dict[str, Proj] = {
    "glm_16k_chunk": Proj("glm_16k_chunk", 4096, 51),
    "glm_decode_8": Proj("glm_decode_8", 8, 52),
    "glm_small": Proj("glm_small", 37, 53),
}


def make_proj(cfg: Proj) -> Dict[str, np.ndarray]:
    """o ~ N(0,1)*0.02 in float32; wv ~ N(0,1)/sqrt(Dl) and wo ~ N(0,1)/sqrt(H*Dv)
    rounded to bf16; x (an output-projection input of its own) ~ N(0,1)*0.1
    rounded to bf16.  Drawn in the order o, wv, wo, x."""
    rng = np.random.default_rng(cfg.seed)
    nrm = lambda *shp: rng.standard_normal(size=shp, dtype=np.float32)
    o = nrm(cfg.T, cfg.H, cfg.Dl) * np.float32(0.02)
    wv = to_bf16_bits(nrm(cfg.H, cfg.Dv, cfg.Dl) * np.float32(1.0 / np.sqrt(cfg.Dl)))
    wo = to_bf16_bits(nrm(cfg.hidden, cfg.H * cfg.Dv) * np.float32(1.0 / np.sqrt(cfg.H * cfg.Dv)))
    x = to_bf16_bits(nrm(cfg.T, cfg.H * cfg.Dv) * np.float32(0.1))
    return {"o": np.ascontiguousarray(o), "wv": wv, "wo": wo, "x": x}


@dataclasses.dataclass(frozen=True)
class Dense:
    """A prefill chunk on the dense masked path, non-absorbed form: L queries
    at positions q_start .. q_start+L-1 over N keys.  Per head the query is
    [no-rope Dn | rope Dr] and kvb holds [no-rope key Dn | value Dv]; the rope
    key is the cache row's columns Dl .. Dl+Dr-1.  The selection is the top_k
    of seeded random indexer scores (GLM: 64 heads, 192 + 64 score dims,
    v_head_dim 256, top_k 2048, dense below 8192 keys of context, chunks of
    4096 tokens)."""
    name: str
    L: int
    N: int
    q_start: int
    seed: int
    H: int = 64
    Dn: int = 192
    Dr: int = 64
    Dv: int = 256
    Dl: int = 512
    top_k: int = 2048


DENSE: Dict[str, Dense] = {
    "glm_8k_chunk": Dense("glm_8k_chunk", 4096, 8192, 4096, 61),
    "glm_4k_first": Dense("glm_4k_first", 4096, 4096, 0, 62),
    "glm_small": Dense("glm_small", 160, 700, 540, 63, top_k=128),
    "tiny": Dense("tiny", 200, 300, 100, 64, H=4, Dn=64, Dr=64, Dv=64, Dl=64, top_k=64),
    "tiny_first": Dense("tiny_first", 150, 150, 0, 65, H=3, Dn=64, Dr=64, Dv=64, Dl=64, top_k=64),
}


def make_dense(cfg: Dense) -> Dict[str, np.ndarray]:
    """q, kvb and the cache rows kv ~ N(0,1) rounded to bf16; indexer scores
    S ~ N(0,1) in float32 for the selection (the causal limit is applied by
    the selection step).  Drawn in the order q, kvb, kv, S."""
    rng = np.random.default_rng(cfg.seed)
    nrm = lambda *shp: rng.standard_normal(size=shp, dtype=np.float32)
    q = to_bf16_bits(nrm(cfg.L, cfg.H, cfg.Dn + cfg.Dr))
    kvb = to_bf16_bits(nrm(cfg.N, cfg.H, cfg.Dn + cfg.Dv))
    kv = to_bf16_bits(nrm(cfg.N, cfg.Dl + cfg.Dr))
    S = nrm(cfg.L, cfg.N)
    return {"q": q, "kvb": kvb, "kv": kv, "S": S}


def make_kvb_weight(cfg: Dense) -> np.ndarray:
    """The kv_b weight [H * (Dn + Dv), Dl] ~ N(0,1)/sqrt(Dl) rounded to bf16,
    from a stream of its own (seed + 1000), so make_dense's draws stay put."""
    rng = np.random.default_rng(cfg.seed + 1000)
    w = rng.standard_normal(size=(cfg.H * (cfg.Dn + cfg.Dv), cfg.Dl), dtype=np.float32)
    return to_bf16_bits(w * np.float32(1.0 / np.sqrt(cfg.Dl)))

