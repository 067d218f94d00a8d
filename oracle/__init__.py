"""ctypes wrapper of the plain C oracle (``dsa_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg import this module.  The HIP library and its binding never
import it.  Arrays are numpy, host memory; bf16 operands are uint16 bit
patterns as drawn by ``workloads``.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "dsa_oracle.h"))):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _configure(lib):
    P = ctypes.c_void_p
    i64, i32, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    lib.oracle_indexer_scores.argtypes = [P, P, P, i64, i64, i64, i32, i32, P, i64, P, i32]
    lib.oracle_topk_select.argtypes = [P, i64, i64, P, i32, P, P, i32]
    lib.oracle_sparse_mla_attn.argtypes = [P, P, P, P, i64, i64, i32, i32, i32, i32, dbl,
                                           P, i64, P, P, i32]
    lib.oracle_prefill_chunk.argtypes = [P, P, P, P, P, i64, i64, i64, i32, i32, i32, i32, i32,
                                         i32, dbl, P, i64, P, P, P, i32]
    lib.oracle_decode_step.argtypes = [P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, dbl,
                                       P, P, P, i32]
    lib.oracle_cache_write.argtypes = [P, P, dbl, P, i64, i64, P, P, P, P, P, i32, i32, i32, i32, i32,
                                       i32, dbl]
    lib.oracle_router_topk.argtypes = [P, P, i64, i32, i32, dbl, dbl, P, P]
    lib.oracle_value_up_proj.argtypes = [P, P, i64, i32, i32, i32, P]
    lib.oracle_o_proj.argtypes = [P, P, i64, i32, i32, P, i64, P]
    lib.oracle_selection_mask.argtypes = [P, P, i64, i32, i64, i64, i64, P]
    lib.oracle_kv_b_proj.argtypes = [P, i32, P, i64, i32, i32, i32, i32, i32, P]
    lib.oracle_q_absorb.argtypes = [P, P, i64, i32, i32, i32, i32, i32, P]
    lib.oracle_dense_masked_attn.argtypes = [P, P, P, P, i64, i64, i32, i32, i32, i32, i32, i32, i64,
                                             dbl, P, i64, P, i32]
    for f in (lib.oracle_indexer_scores, lib.oracle_topk_select, lib.oracle_sparse_mla_attn,
              lib.oracle_prefill_chunk, lib.oracle_decode_step, lib.oracle_cache_write,
              lib.oracle_router_topk, lib.oracle_value_up_proj, lib.oracle_o_proj,
              lib.oracle_selection_mask, lib.oracle_dense_masked_attn, lib.oracle_kv_b_proj,
              lib.oracle_q_absorb):
        f.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = _configure(ctypes.CDLL(build()))
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Run the wrappers against another build of the oracle (the tests use
    this to check that deliberately broken copies fail the pins)."""
    global _lib
    saved = _lib
    _lib = _configure(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


MAX_THREADS = 16   # the CPU share one GPU gets on the measurement hosts


def default_threads() -> int:
    """Host threads for the oracle: the usable cores, at most MAX_THREADS."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_THREADS))


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _rows(rows, L) -> np.ndarray:
    return _c(np.arange(L) if rows is None else rows, np.int64)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError("oracle %s failed with code %d" % (what, rc))


def indexer_scores(qI, kI, w, q_start: int, rows=None, nthreads: Optional[int] = None) -> np.ndarray:
    """Scores [len(rows), N] float32 (-inf on masked keys)."""
    qI, kI, w = _c(qI, np.uint16), _c(kI, np.uint16), _c(w, np.float32)
    L, Hi, Di = qI.shape
    N = kI.shape[0]
    rows = _rows(rows, L)
    S = np.empty((rows.size, N), dtype=np.float32)
    _check(_load().oracle_indexer_scores(_p(qI), _p(kI), _p(w), L, N, q_start, Hi, Di, _p(rows),
                                         rows.size, _p(S), nthreads or default_threads()), "indexer")
    return S


def topk_select(S, pos, top_k: int, nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(idx [rows, top_k] int32 ascending, -1 padded; count [rows] int32)."""
    S = _c(S, np.float32)
    pos = _c(pos, np.int64)
    nrows, N = S.shape
    idx = np.empty((nrows, top_k), dtype=np.int32)
    cnt = np.empty((nrows,), dtype=np.int32)
    _check(_load().oracle_topk_select(_p(S), nrows, N, _p(pos), top_k, _p(idx), _p(cnt),
                                      nthreads or default_threads()), "topk")
    return idx, cnt


def sparse_mla_attn(q, kv, idx, count, d_latent: int, scale: float, rows=None,
                    nthreads: Optional[int] = None, want_lse: bool = False):
    """Attention output [rows, H, Dl] float64 (and lse [rows, H] if asked)."""
    q, kv, idx, count = _c(q, np.uint16), _c(kv, np.uint16), _c(idx, np.int32), _c(count, np.int32)
    L, H, Dqk = q.shape
    N = kv.shape[0]
    top_k = idx.shape[1]
    rows = _rows(rows, L)
    out = np.empty((rows.size, H, d_latent), dtype=np.float64)
    lse = np.empty((rows.size, H), dtype=np.float64) if want_lse else None
    _check(_load().oracle_sparse_mla_attn(_p(q), _p(kv), _p(idx), _p(count), L, N, H, Dqk, d_latent,
                                          top_k, scale, _p(rows), rows.size, _p(out), _p(lse),
                                          nthreads or default_threads()), "attention")
    return (out, lse) if want_lse else out


def prefill_chunk(inp: dict, shape, q_start: int, rows=None, nthreads: Optional[int] = None):
    """(idx [rows, top_k], count [rows], out [rows, H, Dl] float64)."""
    q, qI, w = _c(inp["q"], np.uint16), _c(inp["qI"], np.uint16), _c(inp["w"], np.float32)
    kv, kI = _c(inp["kv"], np.uint16), _c(inp["kI"], np.uint16)
    L, N = q.shape[0], kv.shape[0]
    rows = _rows(rows, L)
    idx = np.empty((rows.size, shape.top_k), dtype=np.int32)
    cnt = np.empty((rows.size,), dtype=np.int32)
    out = np.empty((rows.size, shape.n_heads, shape.d_latent), dtype=np.float64)
    _check(_load().oracle_prefill_chunk(
        _p(q), _p(qI), _p(w), _p(kv), _p(kI), L, N, q_start, shape.n_heads, shape.d_latent,
        shape.d_rope, shape.n_idx_heads, shape.d_idx, shape.top_k, shape.softmax_scale,
        _p(rows), rows.size, _p(idx), _p(cnt), _p(out), nthreads or default_threads()), "prefill")
    return idx, cnt, out


def decode_step(inp: dict, shape, nthreads: Optional[int] = None):
    """(idx [B, top_k] sequence-local key ids, count [B], out [B, H, Dl] float64)."""
    q, qI, w = _c(inp["q"], np.uint16), _c(inp["qI"], np.uint16), _c(inp["w"], np.float32)
    kv, kI = _c(inp["kv"], np.uint16), _c(inp["kI"], np.uint16)
    ctx = _c(inp["ctx"], np.int64)
    B = ctx.size
    idx = np.empty((B, shape.top_k), dtype=np.int32)
    cnt = np.empty((B,), dtype=np.int32)
    out = np.empty((B, shape.n_heads, shape.d_latent), dtype=np.float64)
    _check(_load().oracle_decode_step(
        _p(q), _p(qI), _p(w), _p(kv), _p(kI), B, _p(ctx), shape.n_heads, shape.d_latent,
        shape.d_rope, shape.n_idx_heads, shape.d_idx, shape.top_k, shape.softmax_scale,
        _p(idx), _p(cnt), _p(out), nthreads or default_threads()), "decode")
    return idx, cnt, out


def cache_write(kv_a, norm_w, eps: float, pos, kv_cache, kI_new=None, kI_cache=None, q=None, qI=None,
                *, shape, d_idx_rope: int, theta: float):
    """Upstream cache write; returns new arrays (kv_cache, kI_cache, q, qI),
    the inputs left unchanged (None where not given)."""
    kv_a, norm_w = _c(kv_a, np.uint16), _c(norm_w, np.float32)
    pos = _c(pos, np.int64)
    kv_out = np.array(kv_cache, dtype=np.uint16, copy=True, order="C")
    kI_out = None if kI_cache is None else np.array(kI_cache, dtype=np.uint16, copy=True, order="C")
    kI_new = None if kI_new is None else _c(kI_new, np.uint16)
    q_out = None if q is None else np.array(q, dtype=np.uint16, copy=True, order="C")
    qI_out = None if qI is None else np.array(qI, dtype=np.uint16, copy=True, order="C")
    T, N = pos.size, kv_out.shape[0]
    _check(_load().oracle_cache_write(
        _p(kv_a), _p(norm_w), float(eps), _p(pos), T, N, _p(kv_out), _p(kI_new), _p(kI_out),
        _p(q_out), _p(qI_out), shape.n_heads, shape.d_latent, shape.d_rope, shape.n_idx_heads,
        shape.d_idx, d_idx_rope, float(theta)), "cache write")
    return kv_out, kI_out, q_out, qI_out


ROUTER_MIN_SUM = 6.1e-5   # the clamp on the weight sum (pipeline trace section 8a)


def router_topk(logits, bias, k: int, scale: float, min_sum: float = ROUTER_MIN_SUM):
    """(ids [T, k] int32 by descending selection score, weights [T, k] float64)."""
    logits, bias = _c(logits, np.float32), _c(bias, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    wts = np.empty((T, k), dtype=np.float64)
    _check(_load().oracle_router_topk(_p(logits), _p(bias), T, E, k, float(scale), float(min_sum),
                                      _p(ids), _p(wts)), "router")
    return ids, wts


def value_up_proj(o, wv) -> np.ndarray:
    """out_v [T, H, Dv] bf16 bits from o [T, H, Dl] float32 and wv [H, Dv, Dl] bf16."""
    o, wv = _c(o, np.float32), _c(wv, np.uint16)
    T, H, Dl = o.shape
    Dv = wv.shape[1]
    out = np.empty((T, H, Dv), dtype=np.uint16)
    _check(_load().oracle_value_up_proj(_p(o), _p(wv), T, H, Dl, Dv, _p(out)), "value up-projection")
    return out


def o_proj(x, wo, rows=None) -> np.ndarray:
    """y [len(rows), Nout] float64 from x [T, Kin] bf16 and wo [Nout, Kin] bf16."""
    x, wo = _c(x, np.uint16), _c(wo, np.uint16)
    T, Kin = x.shape
    Nout = wo.shape[0]
    rows = _rows(rows, T)
    y = np.empty((rows.size, Nout), dtype=np.float64)
    _check(_load().oracle_o_proj(_p(x), _p(wo), T, Kin, Nout, _p(rows), rows.size, _p(y)), "o_proj")
    return y


def mask_words(N: int) -> int:
    """Words per mask row: the keys rounded up to a whole 64-key tile."""
    return 2 * ((N + 63) // 64)


def selection_mask(idx, count, N: int, q_start: int, W: Optional[int] = None) -> np.ndarray:
    """Boolean selection mask [L, W] uint32: bit j % 32 of word j // 32 is set
    iff key j is selected, in [0, N) and causal for the query."""
    idx, count = _c(idx, np.int32), _c(count, np.int32)
    L, top_k = idx.shape
    W = mask_words(N) if W is None else W
    mask = np.empty((L, W), dtype=np.uint32)
    _check(_load().oracle_selection_mask(_p(idx), _p(count), L, top_k, N, q_start, W, _p(mask)), "mask")
    return mask


def dense_masked_attn(q, kvb, kv, mask, d_nope: int, d_rope: int, d_v: int, rope_col: int,
                      scale: float, rows=None, nthreads: Optional[int] = None) -> np.ndarray:
    """Non-absorbed attention under a boolean mask: out [rows, H, d_v] float64."""
    q, kvb, kv, mask = _c(q, np.uint16), _c(kvb, np.uint16), _c(kv, np.uint16), _c(mask, np.uint32)
    L, H, Dq = q.shape
    N, Dc = kv.shape
    assert Dq == d_nope + d_rope and kvb.shape == (N, H, d_nope + d_v) and mask.shape[0] == L
    rows = _rows(rows, L)
    out = np.empty((rows.size, H, d_v), dtype=np.float64)
    _check(_load().oracle_dense_masked_attn(_p(q), _p(kvb), _p(kv), _p(mask), L, N, H, d_nope, d_rope, d_v,
                                            Dc, rope_col, mask.shape[1], scale, _p(rows), rows.size, _p(out),
                                            nthreads or default_threads()), "dense attention")
    return out


def q_absorb(q, w, d_latent: int, d_nope: int, d_v: int) -> np.ndarray:
    """The absorbed query [T, H, d_latent + d_rope] as bf16 bits: each head's
    no-rope query times the key block of the kv_b weight w [H * (d_nope +
    d_v), d_latent], the rope part copied (pipeline trace, section 6)."""
    q, w = _c(q, np.uint16), _c(w, np.uint16)
    T, H, qc = q.shape
    Dr = qc - d_nope
    assert Dr >= 0 and w.shape == (H * (d_nope + d_v), d_latent)
    out = np.empty((T, H, d_latent + Dr), dtype=np.uint16)
    _check(_load().oracle_q_absorb(_p(q), _p(w), T, H, d_nope, Dr, d_latent, d_v, _p(out)), "q_absorb")
    return out


def kv_b_proj(kv, w, H: int, d_latent: int, d_nope: int, d_v: int, values_f16: bool) -> np.ndarray:
    """kvb [N, H, d_nope + d_v] as uint16 bits: bf16 no-rope keys, and values
    in bf16 or (values_f16) fp16."""
    kv, w = _c(kv, np.uint16), _c(w, np.uint16)
    N, kv_cols = kv.shape
    assert w.shape == (H * (d_nope + d_v), d_latent)
    out = np.empty((N, H, d_nope + d_v), dtype=np.uint16)
    _check(_load().oracle_kv_b_proj(_p(kv), kv_cols, _p(w), N, H, d_latent, d_nope, d_v, int(values_f16), _p(out)),
           "kv_b")
    return out

