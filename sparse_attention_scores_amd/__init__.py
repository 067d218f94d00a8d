"""Python binding of the MI355X DSA core (``libdsa.so``, C ABI in include/dsa.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, checks dtype / device / contiguity, and passes their data
pointers and the current HIP stream to the C function of the same name.
Every step of the path runs in the library's HIP kernels; there is no
fallback.  If the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

from . import build as _build

__all__ = [
    "DsaError", "Shape", "GLM", "TINY", "lib",
    "dsa_indexer_scores", "dsa_topk_select", "dsa_sparse_mla_attn", "dsa_latent_to_f16",
    "dsa_sparse_mla_attn_f16", "dsa_prefill_workspace_bytes", "dsa_prefill_chunk",
    "dsa_decode_workspace_bytes", "dsa_decode_step", "dsa_decode_step_noalloc", "dsa_cache_write",
    "dsa_router_topk", "dsa_value_up_proj", "dsa_o_proj", "dsa_selection_mask", "dsa_dense_masked_attn",
    "dsa_dense_masked_attn_f16", "dsa_values_to_f16", "dsa_kv_b_proj", "dsa_q_absorb", "dsa_absorb_weight",
    "dsa_status_string",
    "EXPORTED_SYMBOLS", "DECODE_STATIC_SCRATCH_BYTES",
]

EXPORTED_SYMBOLS = (
    "dsa_status_string", "dsa_indexer_scores", "dsa_topk_select", "dsa_sparse_mla_attn",
    "dsa_latent_to_f16", "dsa_sparse_mla_attn_f16", "dsa_prefill_workspace_bytes", "dsa_prefill_chunk",
    "dsa_decode_workspace_bytes", "dsa_decode_step", "dsa_decode_step_noalloc", "dsa_cache_write",
    "dsa_router_topk", "dsa_value_up_proj", "dsa_o_proj", "dsa_selection_mask", "dsa_dense_masked_attn",
    "dsa_dense_masked_attn_f16", "dsa_values_to_f16", "dsa_kv_b_proj", "dsa_q_absorb", "dsa_absorb_weight",
)

DECODE_STATIC_SCRATCH_BYTES = 32 << 20   # DSA_DECODE_STATIC_SCRATCH_BYTES in include/dsa.h


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s: %s" % (fn, msg))
        self.status = status


class Shape(ctypes.Structure):
    """dsa_shape: (n_heads, d_latent, d_rope, n_idx_heads, d_idx, top_k, softmax_scale)."""
    _fields_ = [("n_heads", ctypes.c_int32), ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("n_idx_heads", ctypes.c_int32), ("d_idx", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]

    @classmethod
    def of(cls, s) -> "Shape":
        """From any object with the same attribute names (e.g. workloads.Shape)."""
        if isinstance(s, cls):
            return s
        return cls(s.n_heads, s.d_latent, s.d_rope, s.n_idx_heads, s.d_idx, s.top_k, s.softmax_scale)

    @property
    def d_qk(self) -> int:
        return self.d_latent + self.d_rope


GLM = Shape(64, 512, 64, 32, 128, 2048, 1.0 / 16)
TINY = Shape(4, 64, 16, 4, 32, 32, 1.0 / 16)


def _load() -> ctypes.CDLL:
    if not os.path.exists(_build.LIB):
        _build.build()
    L = ctypes.CDLL(_build.LIB)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    SP = ctypes.POINTER(Shape)
    sig = {
        "dsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "dsa_indexer_scores": (ctypes.c_int, [SP, P, P, P, i32, i32, i64, P, P]),
        "dsa_topk_select": (ctypes.c_int, [SP, P, i32, i32, i64, P, P, P]),
        "dsa_sparse_mla_attn": (ctypes.c_int, [SP, P, P, P, P, i32, i32, P, P, P]),
        "dsa_latent_to_f16": (ctypes.c_int, [SP, P, i32, P, P]),
        "dsa_sparse_mla_attn_f16": (ctypes.c_int, [SP, P, P, P, P, i32, i32, P, P, P]),
        "dsa_prefill_workspace_bytes": (sz, [SP, i32, i32, i64]),
        "dsa_prefill_chunk": (ctypes.c_int, [SP, P, P, P, P, P, i32, i32, i64, P, P, P, P, sz, P]),
        "dsa_decode_workspace_bytes": (sz, [SP, i32, P]),
        "dsa_decode_step": (ctypes.c_int, [SP, i32, P, P, P, P, P, P, P, P, P, P, sz, P]),
        "dsa_decode_step_noalloc": (ctypes.c_int, [SP, i32, P, P, P, P, P, P, P, P, P, P]),
        "dsa_cache_write": (ctypes.c_int, [SP, P, P, ctypes.c_float, P, i32, i32, P, P, P, P, P, i32,
                                           ctypes.c_float, P]),
        "dsa_router_topk": (ctypes.c_int, [P, P, i32, i32, i32, ctypes.c_float, P, P, P]),
        "dsa_value_up_proj": (ctypes.c_int, [SP, P, P, i32, i32, P, P]),
        "dsa_o_proj": (ctypes.c_int, [P, P, i32, i32, i32, P, P]),
        "dsa_selection_mask": (ctypes.c_int, [P, P, i32, i32, i32, i32, i32, P, P]),
        "dsa_dense_masked_attn": (ctypes.c_int, [P, P, P, i32, i32, P, i32, i32, i32, i32, i32, i32, i32, i32,
                                                 ctypes.c_float, P, P]),
        "dsa_dense_masked_attn_f16": (ctypes.c_int, [P, P, P, P, i32, i32, P, i32, i32, i32, i32, i32, i32, i32,
                                                     i32, ctypes.c_float, P, P]),
        "dsa_values_to_f16": (ctypes.c_int, [P, i32, i32, i32, i32, P, P]),
        "dsa_kv_b_proj": (ctypes.c_int, [P, i32, P, i32, i32, i32, i32, i32, P, P, P]),
        "dsa_q_absorb": (ctypes.c_int, [P, P, i32, i32, i32, i32, i32, P, P]),
        "dsa_absorb_weight": (ctypes.c_int, [P, i32, i32, i32, i32, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    return L


lib = _load()


def dsa_status_string(status: int) -> str:
    return lib.dsa_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise DsaError(fn, status, dsa_status_string(status))


def _ptr(t: Optional[torch.Tensor], dtype: torch.dtype, name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.dtype != dtype:
        raise TypeError("%s must be a %s tensor" % (name, dtype))
    if not t.is_cuda:
        raise ValueError("%s must live on the GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# bf16 operands travel as their 16-bit patterns: int16/uint16/bfloat16 tensors
def _bits(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if t.dtype not in (torch.bfloat16, torch.float16, torch.int16, torch.uint16):
        raise TypeError("%s must hold 16-bit patterns (bfloat16/float16/int16/uint16)" % name)
    return _ptr(t, t.dtype, name)


def dsa_indexer_scores(shape, qI, kI, w, L: int, N: int, q_start: int, S, stream=None) -> None:
    sh = Shape.of(shape)
    _check("dsa_indexer_scores", lib.dsa_indexer_scores(
        ctypes.byref(sh), _bits(qI, "qI"), _bits(kI, "kI"), _ptr(w, torch.float32, "w"),
        L, N, q_start, _ptr(S, torch.float32, "S"), _stream(stream)))


def dsa_topk_select(shape, S, L: int, N: int, q_start: int, idx, count, stream=None) -> None:
    sh = Shape.of(shape)
    _check("dsa_topk_select", lib.dsa_topk_select(
        ctypes.byref(sh), _ptr(S, torch.float32, "S"), L, N, q_start,
        _ptr(idx, torch.int32, "idx"), _ptr(count, torch.int32, "count"), _stream(stream)))


def dsa_sparse_mla_attn(shape, q, kv, idx, count, L: int, N: int, out, lse=None, stream=None) -> None:
    sh = Shape.of(shape)
    _check("dsa_sparse_mla_attn", lib.dsa_sparse_mla_attn(
        ctypes.byref(sh), _bits(q, "q"), _bits(kv, "kv"), _ptr(idx, torch.int32, "idx"),
        _ptr(count, torch.int32, "count"), L, N, _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse"), _stream(stream)))


def dsa_latent_to_f16(shape, kv, N: int, kv16, stream=None) -> None:
    sh = Shape.of(shape)
    _check("dsa_latent_to_f16", lib.dsa_latent_to_f16(ctypes.byref(sh), _bits(kv, "kv"), N, _bits(kv16, "kv16"),
                                                      _stream(stream)))


def dsa_sparse_mla_attn_f16(shape, q, kv16, idx, count, L: int, N: int, out, lse=None, stream=None) -> None:
    sh = Shape.of(shape)
    _check("dsa_sparse_mla_attn_f16", lib.dsa_sparse_mla_attn_f16(
        ctypes.byref(sh), _bits(q, "q"), _bits(kv16, "kv16"), _ptr(idx, torch.int32, "idx"),
        _ptr(count, torch.int32, "count"), L, N, _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse"), _stream(stream)))


def dsa_prefill_workspace_bytes(shape, L: int, N: int, q_start: int) -> int:
    return int(lib.dsa_prefill_workspace_bytes(ctypes.byref(Shape.of(shape)), L, N, q_start))


def dsa_prefill_chunk(shape, q, qI, w, kv, kI, L: int, N: int, q_start: int, out, idx_out=None,
                      count_out=None, ws=None, stream=None) -> None:
    sh = Shape.of(shape)
    ws_ptr, ws_bytes = (None, 0) if ws is None else (_ptr(ws, torch.uint8, "ws"), ws.numel())
    _check("dsa_prefill_chunk", lib.dsa_prefill_chunk(
        ctypes.byref(sh), _bits(q, "q"), _bits(qI, "qI"), _ptr(w, torch.float32, "w"), _bits(kv, "kv"),
        _bits(kI, "kI"), L, N, q_start, _ptr(out, torch.float32, "out"),
        _ptr(idx_out, torch.int32, "idx_out"), _ptr(count_out, torch.int32, "count_out"),
        ws_ptr, ws_bytes, _stream(stream)))


def _ctx_array(ctx: Sequence[int]):
    arr = (ctypes.c_int64 * len(ctx))(*[int(c) for c in ctx])
    return arr


def dsa_decode_workspace_bytes(shape, ctx: Sequence[int]) -> int:
    arr = _ctx_array(ctx)
    return int(lib.dsa_decode_workspace_bytes(ctypes.byref(Shape.of(shape)), len(ctx),
                                              ctypes.cast(arr, ctypes.c_void_p)))


def dsa_decode_step(shape, ctx: Sequence[int], q, qI, w, kv, kI, out, idx_out=None, count_out=None,
                    ws=None, stream=None) -> None:
    sh = Shape.of(shape)
    arr = _ctx_array(ctx)
    ws_ptr, ws_bytes = (None, 0) if ws is None else (_ptr(ws, torch.uint8, "ws"), ws.numel())
    _check("dsa_decode_step", lib.dsa_decode_step(
        ctypes.byref(sh), len(ctx), ctypes.cast(arr, ctypes.c_void_p), _bits(q, "q"), _bits(qI, "qI"),
        _ptr(w, torch.float32, "w"), _bits(kv, "kv"), _bits(kI, "kI"), _ptr(out, torch.float32, "out"),
        _ptr(idx_out, torch.int32, "idx_out"), _ptr(count_out, torch.int32, "count_out"),
        ws_ptr, ws_bytes, _stream(stream)))


def dsa_decode_step_noalloc(shape, ctx: Sequence[int], q, qI, w, kv, kI, out, idx_out=None, count_out=None,
                            stream=None) -> None:
    sh = Shape.of(shape)
    arr = _ctx_array(ctx)
    _check("dsa_decode_step_noalloc", lib.dsa_decode_step_noalloc(
        ctypes.byref(sh), len(ctx), ctypes.cast(arr, ctypes.c_void_p), _bits(q, "q"), _bits(qI, "qI"),
        _ptr(w, torch.float32, "w"), _bits(kv, "kv"), _bits(kI, "kI"), _ptr(out, torch.float32, "out"),
        _ptr(idx_out, torch.int32, "idx_out"), _ptr(count_out, torch.int32, "count_out"), _stream(stream)))


def dsa_cache_write(shape, kv_a, norm_w, eps: float, pos, T: int, N: int, kv, kI_new=None, kI=None,
                    q=None, qI=None, d_idx_rope: int = 64, rope_theta: float = 10000.0,
                    stream=None) -> None:
    sh = Shape.of(shape)
    _check("dsa_cache_write", lib.dsa_cache_write(
        ctypes.byref(sh), _bits(kv_a, "kv_a"), _ptr(norm_w, torch.float32, "norm_w"), float(eps),
        _ptr(pos, torch.int32, "pos"), T, N, _bits(kv, "kv"), _bits(kI_new, "kI_new"), _bits(kI, "kI"),
        _bits(q, "q"), _bits(qI, "qI"), d_idx_rope, float(rope_theta), _stream(stream)))


def dsa_router_topk(logits, bias, T: int, n_experts: int, k: int, routed_scale: float, ids, weights,
                    stream=None) -> None:
    _check("dsa_router_topk", lib.dsa_router_topk(
        _ptr(logits, torch.float32, "logits"), _ptr(bias, torch.float32, "bias"), T, n_experts, k,
        float(routed_scale), _ptr(ids, torch.int32, "ids"), _ptr(weights, torch.float32, "weights"),
        _stream(stream)))


def dsa_value_up_proj(shape, o, wv, T: int, d_v: int, out_v, stream=None) -> None:
    sh = Shape.of(shape)
    _check("dsa_value_up_proj", lib.dsa_value_up_proj(
        ctypes.byref(sh), _ptr(o, torch.float32, "o"), _bits(wv, "wv"), T, d_v, _bits(out_v, "out_v"),
        _stream(stream)))


def dsa_o_proj(x, wo, T: int, k_in: int, n_out: int, y, stream=None) -> None:
    _check("dsa_o_proj", lib.dsa_o_proj(_bits(x, "x"), _bits(wo, "wo"), T, k_in, n_out,
                                        _ptr(y, torch.float32, "y"), _stream(stream)))


def mask_words(N: int) -> int:
    """Words per selection-mask row: N keys rounded up to whole 64-key tiles."""
    return 2 * ((N + 63) // 64)


def dsa_selection_mask(idx, count, L: int, top_k: int, N: int, q_start: int, mask, stream=None) -> None:
    _check("dsa_selection_mask", lib.dsa_selection_mask(
        _ptr(idx, torch.int32, "idx"), _ptr(count, torch.int32, "count"), L, top_k, N, q_start,
        mask.shape[1] if mask is not None and mask.dim() == 2 else 0, _ptr(mask, torch.int32, "mask"),
        _stream(stream)))


def dsa_dense_masked_attn(q, kvb, kv, kv_cols: int, rope_col: int, mask, L: int, N: int, q_start: int, H: int,
                          d_nope: int, d_rope: int, d_v: int, scale: float, out, stream=None) -> None:
    _check("dsa_dense_masked_attn", lib.dsa_dense_masked_attn(
        _bits(q, "q"), _bits(kvb, "kvb"), _bits(kv, "kv"), kv_cols, rope_col, _ptr(mask, torch.int32, "mask"),
        mask.shape[1] if mask is not None and mask.dim() == 2 else 0, L, N, q_start, H, d_nope, d_rope, d_v,
        scale, _ptr(out, torch.float32, "out"), _stream(stream)))


def vt_keys(N: int) -> int:
    """Key stride of the fp16 value form vt [H, d_v, Np]: N rounded up to 64."""
    return 64 * ((N + 63) // 64)


def dsa_dense_masked_attn_f16(q, kvb, vt, kv, kv_cols: int, rope_col: int, mask, L: int, N: int, q_start: int,
                              H: int, d_nope: int, d_rope: int, d_v: int, scale: float, out, stream=None) -> None:
    _check("dsa_dense_masked_attn_f16", lib.dsa_dense_masked_attn_f16(
        _bits(q, "q"), _bits(kvb, "kvb"), _bits(vt, "vt"), _bits(kv, "kv"), kv_cols, rope_col,
        _ptr(mask, torch.int32, "mask"),
        mask.shape[1] if mask is not None and mask.dim() == 2 else 0, L, N, q_start, H, d_nope, d_rope, d_v,
        scale, _ptr(out, torch.float32, "out"), _stream(stream)))


def dsa_values_to_f16(kvb, N: int, H: int, d_nope: int, d_v: int, vt, stream=None) -> None:
    _check("dsa_values_to_f16", lib.dsa_values_to_f16(_bits(kvb, "kvb"), N, H, d_nope, d_v, _bits(vt, "vt"),
                                                      _stream(stream)))


def dsa_absorb_weight(wkvb, H: int, d_nope: int, d_v: int, d_latent: int, wk_t, stream=None) -> None:
    _check("dsa_absorb_weight", lib.dsa_absorb_weight(_bits(wkvb, "wkvb"), H, d_nope, d_v, d_latent,
                                                      _bits(wk_t, "wk_t"), _stream(stream)))


def dsa_q_absorb(q, wk_t, T: int, H: int, d_nope: int, d_rope: int, d_latent: int, q_abs, stream=None) -> None:
    _check("dsa_q_absorb", lib.dsa_q_absorb(_bits(q, "q"), _bits(wk_t, "wk_t"), T, H, d_nope, d_rope, d_latent,
                                            _bits(q_abs, "q_abs"), _stream(stream)))


def dsa_kv_b_proj(kv, kv_cols: int, wkvb, N: int, H: int, d_latent: int, d_nope: int, d_v: int, kvb, vt=None,
                  stream=None) -> None:
    _check("dsa_kv_b_proj", lib.dsa_kv_b_proj(_bits(kv, "kv"), kv_cols, _bits(wkvb, "wkvb"), N, H, d_latent, d_nope,
                                              d_v, _bits(kvb, "kvb"), _bits(vt, "vt"), _stream(stream)))

