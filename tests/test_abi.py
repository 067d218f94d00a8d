"""Host-only checks of the C ABI: the library loads, exports every function
include/dsa.h declares, and rejects bad arguments before any launch (these
run without a GPU: validation happens before the first HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

dsa = pytest.importorskip("sparse_attention_scores_amd")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, -1, -2, -3, -4


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 22, names
    assert sorted(dsa.EXPORTED_SYMBOLS) == names
    raw = ctypes.CDLL(dsa._build.LIB)
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings():
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR):
        assert dsa.dsa_status_string(code).startswith("DSA_")
    assert "unknown" in dsa.dsa_status_string(7)


def fake(addr=0x1000):
    return ctypes.c_void_p(addr)


def test_shape_validation():
    L = dsa.lib
    bad = dsa.Shape(64, 512, 64, 32, 128, 2048, 1.0 / 16)
    bad.n_heads = 8                       # not a supported head count
    assert L.dsa_indexer_scores(ctypes.byref(bad), fake(), fake(), fake(), 4, 8, 0, fake(), None) == UNSUPPORTED
    big = dsa.Shape(64, 512, 64, 32, 128, 4096, 1.0 / 16)
    assert L.dsa_topk_select(ctypes.byref(big), fake(), 4, 8, 0, fake(), fake(), None) == UNSUPPORTED
    neg = dsa.Shape(64, 512, 64, 32, 128, 0, 1.0 / 16)
    assert L.dsa_topk_select(ctypes.byref(neg), fake(), 4, 8, 0, fake(), fake(), None) == INVALID
    nan = dsa.Shape(64, 512, 64, 32, 128, 2048, float("nan"))
    assert L.dsa_sparse_mla_attn(ctypes.byref(nan), fake(), fake(), fake(), fake(), 1, 1, fake(), None, None) == INVALID
    assert L.dsa_indexer_scores(None, fake(), fake(), fake(), 4, 8, 0, fake(), None) == INVALID


def test_pointer_and_size_validation():
    L, sh = dsa.lib, ctypes.byref(dsa.GLM)
    assert L.dsa_indexer_scores(sh, None, fake(), fake(), 4, 8, 0, fake(), None) == INVALID
    assert L.dsa_indexer_scores(sh, fake(0x1008), fake(), fake(), 4, 8, 0, fake(), None) == INVALID  # misaligned
    assert L.dsa_indexer_scores(sh, fake(), fake(), fake(), 0, 8, 0, fake(), None) == INVALID        # L = 0
    assert L.dsa_indexer_scores(sh, fake(), fake(), fake(), 4, 8, 5, fake(), None) == INVALID        # q_start+L > N
    assert L.dsa_indexer_scores(sh, fake(), fake(), fake(), 4, 8, -1, fake(), None) == INVALID
    assert L.dsa_topk_select(sh, fake(), 4, 262145, 262141, fake(), fake(), None) == UNSUPPORTED  # > 262144 keys
    assert L.dsa_sparse_mla_attn(sh, fake(), fake(), None, fake(), 1, 1, fake(), None, None) == INVALID
    assert L.dsa_sparse_mla_attn(sh, fake(), fake(), fake(), fake(), 1, 1, fake(), fake(0x1004), None) == INVALID


def test_prefill_workspace_and_validation():
    L, sh = dsa.lib, ctypes.byref(dsa.GLM)
    assert dsa.dsa_prefill_workspace_bytes(dsa.GLM, 4096, 16384, 12288) > 4096 * 16384 * 4
    # the first chunk only scores queries past position 2047
    small = dsa.dsa_prefill_workspace_bytes(dsa.GLM, 4096, 4096, 0)
    idx_bytes = 4096 * 2048 * 4
    assert 2048 * 4096 * 4 + idx_bytes <= small < 4096 * 4096 * 4 + idx_bytes
    assert dsa.dsa_prefill_workspace_bytes(dsa.GLM, 4096, 16000, 12288) == 0      # N != q_start + L
    args = [fake()] * 5
    rc = L.dsa_prefill_chunk(sh, *args, 16, 16, 0, fake(), None, None, fake(), 0, None)
    assert rc == WORKSPACE
    rc = L.dsa_prefill_chunk(sh, *args, 16, 17, 0, fake(), None, None, fake(), 1 << 30, None)
    assert rc == INVALID
    rc = L.dsa_prefill_chunk(sh, None, *args[1:], 16, 16, 0, fake(), None, None, fake(), 1 << 30, None)
    assert rc == INVALID


def test_decode_workspace_and_validation():
    L, sh = dsa.lib, ctypes.byref(dsa.GLM)
    ctx = [4096, 8192, 16384, 32768, 65536, 65536, 16384, 4096]
    ws = dsa.dsa_decode_workspace_bytes(dsa.GLM, ctx)
    assert ws >= sum(ctx) * 4
    assert dsa.dsa_decode_workspace_bytes(dsa.GLM, [0, 5]) == 0
    assert dsa.dsa_decode_workspace_bytes(dsa.GLM, [262145]) == 0
    assert dsa.dsa_decode_workspace_bytes(dsa.GLM, [262144]) > 0
    arr = (ctypes.c_int64 * 2)(100, 0)
    rc = L.dsa_decode_step(sh, 2, ctypes.cast(arr, ctypes.c_void_p), *([fake()] * 6), None, None,
                           fake(), 1 << 30, None)
    assert rc == INVALID
    arr = (ctypes.c_int64 * 1)(100)
    rc = L.dsa_decode_step(sh, 1, ctypes.cast(arr, ctypes.c_void_p), *([fake()] * 6), None, None,
                           fake(), 16, None)
    assert rc == WORKSPACE
    # batches past 128 sequences run in groups: the workspace covers the largest group
    assert dsa.dsa_decode_workspace_bytes(dsa.GLM, [10] * 200) == dsa.dsa_decode_workspace_bytes(dsa.GLM, [10] * 128)
    ws_a, ws_b = dsa.dsa_decode_workspace_bytes(dsa.GLM, [10] * 128), dsa.dsa_decode_workspace_bytes(dsa.GLM, [65536] * 3)
    assert dsa.dsa_decode_workspace_bytes(dsa.GLM, [10] * 128 + [65536] * 3) == max(ws_a, ws_b)
    many = (ctypes.c_int64 * 16385)(*([10] * 16385))
    rc = L.dsa_decode_step(sh, 16385, ctypes.cast(many, ctypes.c_void_p), *([fake()] * 6), None, None,
                           fake(), 1 << 30, None)
    assert rc == UNSUPPORTED


def test_cache_write_validation():
    L, sh = dsa.lib, ctypes.byref(dsa.GLM)
    f = ctypes.c_float
    def cw(kv_a=None, norm_w=None, pos=None, kv=None, kI_new=None, kI=None, q=None, qI=None, T=4, N=8,
           d_idx_rope=64, theta=10000.0, eps=1e-6):
        return L.dsa_cache_write(sh, kv_a or fake(), norm_w or fake(), f(eps), pos or fake(), T, N,
                                 kv or fake(), kI_new, kI, q, qI, d_idx_rope, f(theta), None)
    assert cw(kv_a=fake(0x1008)) == INVALID                     # misaligned
    assert cw(norm_w=fake(0x1002)) == INVALID                   # norm weight not 4-byte aligned
    assert cw(kI_new=fake()) == INVALID                         # key without its cache
    assert cw(T=-1) == INVALID
    assert cw(N=0) == INVALID
    assert cw(theta=0.0) == INVALID and cw(theta=float("inf")) == INVALID
    assert cw(eps=-1.0) == INVALID and cw(eps=float("nan")) == INVALID
    assert cw(d_idx_rope=130) == INVALID and cw(d_idx_rope=-2) == INVALID
    assert cw(d_idx_rope=6) == UNSUPPORTED                      # not a multiple of 8
    assert cw(T=0) == OK                                        # nothing to do, nothing enqueued
    assert L.dsa_cache_write(None, fake(), fake(), f(0), fake(), 1, 1, fake(), None, None, None, None,
                             64, f(1e4), None) == INVALID


def test_router_validation():
    L = dsa.lib
    f = ctypes.c_float
    def rt(logits=None, bias=None, ids=None, w=None, T=4, E=256, k=8, scale=2.5):
        return L.dsa_router_topk(logits or fake(), bias or fake(), T, E, k, f(scale), ids or fake(),
                                 w or fake(), None)
    assert rt(logits=fake(0x1004)) == INVALID          # logits not 16-byte aligned
    assert rt(bias=fake(0x1002)) == INVALID
    assert rt(T=-1) == INVALID and rt(k=0) == INVALID and rt(k=300) == INVALID
    assert rt(scale=float("nan")) == INVALID
    assert rt(E=96, k=8) == UNSUPPORTED and rt(E=256, k=33) == UNSUPPORTED
    assert rt(T=0) == OK
    assert L.dsa_router_topk(None, fake(), 1, 256, 8, f(2.5), fake(), fake(), None) == INVALID


def test_projection_validation():
    L, sh = dsa.lib, ctypes.byref(dsa.GLM)
    assert L.dsa_value_up_proj(sh, fake(0x1004), fake(), 4, 256, fake(), None) == INVALID
    assert L.dsa_value_up_proj(sh, fake(), fake(), -1, 256, fake(), None) == INVALID
    assert L.dsa_value_up_proj(sh, fake(), fake(), 4, 128, fake(), None) == UNSUPPORTED
    assert L.dsa_value_up_proj(sh, fake(), fake(), 0, 256, fake(), None) == OK
    assert L.dsa_o_proj(fake(), fake(), 4, 16384, 6144, None, None) == INVALID
    assert L.dsa_o_proj(fake(), fake(), 4, 100, 6144, fake(), None) == UNSUPPORTED
    assert L.dsa_o_proj(fake(), fake(), 4, 16384, 6000, fake(), None) == UNSUPPORTED
    assert L.dsa_o_proj(fake(), fake(), 0, 16384, 6144, fake(), None) == OK


def test_dense_validation():
    L = dsa.lib
    W = dsa.mask_words(300)
    assert W == 10
    # selection mask
    assert L.dsa_selection_mask(None, fake(), 8, 64, 300, 0, W, fake(), None) == INVALID
    assert L.dsa_selection_mask(fake(), fake(), 8, 64, 300, 0, W - 1, fake(), None) == INVALID
    assert L.dsa_selection_mask(fake(), fake(), 8, 64, 300, -1, W, fake(), None) == INVALID
    assert L.dsa_selection_mask(fake(), fake(), 8, 0, 300, 0, W, fake(), None) == INVALID
    assert L.dsa_selection_mask(fake(), fake(), 8, 64, 600000, 0, 2 * 9375, fake(), None) == UNSUPPORTED
    assert L.dsa_selection_mask(fake(), fake(), 0, 64, 300, 0, W, fake(), None) == OK
    # dense attention: (Dn, Dr, Dv) = (64, 64, 64), rope at column 64 of 128
    args = lambda **k: [k.get("q", fake()), k.get("kvb", fake()), k.get("kv", fake()), k.get("kv_cols", 128),
                        k.get("rope_col", 64), k.get("mask", fake()), k.get("W", W), k.get("Lq", 8),
                        k.get("N", 300), k.get("q_start", 0), k.get("H", 4), k.get("dn", 64), k.get("dr", 64),
                        k.get("dv", 64), k.get("scale", 0.0625), k.get("out", fake()), None]
    f = L.dsa_dense_masked_attn
    assert f(*args(Lq=0)) == OK
    assert f(*args(q=fake(0x1008), Lq=0)) == INVALID
    assert f(*args(mask=fake(0x1002), Lq=0)) == INVALID
    assert f(*args(out=None)) == INVALID
    assert f(*args(W=W - 2)) == INVALID
    assert f(*args(rope_col=72)) == INVALID
    assert f(*args(kv_cols=132)) == INVALID
    assert f(*args(N=0)) == INVALID
    assert f(*args(H=0)) == INVALID
    assert f(*args(q_start=-1)) == INVALID
    assert f(*args(scale=0.0)) == INVALID
    assert f(*args(scale=float("inf"))) == INVALID
    assert f(*args(dn=48, dr=16)) == UNSUPPORTED
    assert f(*args(dn=192, dr=64, dv=256, kv_cols=576, rope_col=512, Lq=0)) == OK
    g = L.dsa_dense_masked_attn_f16
    gargs = lambda **kw: args(**kw)[:2] + [kw.get("vt", fake())] + args(**kw)[2:]
    assert g(*gargs(Lq=0)) == OK
    assert g(*gargs(vt=None)) == INVALID
    assert g(*gargs(vt=fake(0x1008), Lq=0)) == INVALID
    assert g(*gargs(W=W - 2)) == INVALID
    assert g(*gargs(dn=32, dr=32)) == UNSUPPORTED
    v = L.dsa_values_to_f16
    assert v(None, 8, 4, 64, 64, fake(), None) == INVALID
    assert v(fake(), 8, 4, 64, 64, None, None) == INVALID
    assert v(fake(0x1008), 8, 4, 64, 64, fake(), None) == INVALID
    assert v(fake(), 8, 4, 60, 64, fake(), None) == INVALID
    assert v(fake(), 8, 0, 64, 64, fake(), None) == INVALID
    assert v(fake(), 8, 4, 64, 128, fake(), None) == UNSUPPORTED
    assert v(fake(), 0, 4, 192, 256, fake(), None) == OK
    k = L.dsa_kv_b_proj
    assert k(fake(), 576, fake(), 0, 64, 512, 192, 256, fake(), fake(), None) == OK
    assert k(fake(), 576, fake(), 0, 64, 512, 192, 256, fake(), None, None) == OK
    assert k(None, 576, fake(), 8, 64, 512, 192, 256, fake(), fake(), None) == INVALID
    assert k(fake(), 576, fake(), 8, 64, 512, 192, 256, fake(), fake(0x1008), None) == INVALID
    assert k(fake(), 576, fake(), 8, 64, 640, 192, 256, fake(), fake(), None) == INVALID
    assert k(fake(), 572, fake(), 8, 64, 512, 192, 256, fake(), fake(), None) == INVALID
    assert k(fake(), 576, fake(), 8, 64, 480, 192, 256, fake(), fake(), None) == UNSUPPORTED
    assert k(fake(), 576, fake(), 8, 3, 512, 192, 256, fake(), fake(), None) == UNSUPPORTED
    a = L.dsa_q_absorb
    assert a(fake(), fake(), 0, 64, 192, 64, 512, fake(), None) == OK            # T = 0: nothing enqueued
    assert a(None, fake(), 8, 64, 192, 64, 512, fake(), None) == INVALID
    assert a(fake(), fake(), 8, 64, 192, 64, 512, fake(0x1008), None) == INVALID
    assert a(fake(), fake(), 8, 0, 192, 64, 512, fake(), None) == INVALID
    assert a(fake(), fake(), 8, 64, 160, 64, 512, fake(), None) == UNSUPPORTED   # d_nope % 64
    assert a(fake(), fake(), 8, 64, 192, 64, 384, fake(), None) == UNSUPPORTED   # d_latent % 256
    assert a(fake(), fake(), 8, 64, 192, 60, 512, fake(), None) == UNSUPPORTED   # d_rope % 8
    assert a(fake(), fake(), 1 << 20, 64, 192, 64, 512, fake(), None) == UNSUPPORTED   # 32-bit row offsets
    aw = L.dsa_absorb_weight
    assert aw(None, 64, 192, 256, 512, fake(), None) == INVALID
    assert aw(fake(), 0, 192, 256, 512, fake(), None) == INVALID
