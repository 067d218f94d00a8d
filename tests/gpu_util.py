"""Helpers shared by the GPU tests (no method arithmetic here)."""
import sys

import numpy as np
import pytest

# Attention tolerance: max over (query, head) rows of max_d |o - r| / max_d |r|.
ATTN_TOL = 2e-3


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


requires_gpu = pytest.mark.skipif(not gpu_available(), reason="needs a GPU")


def say(*a):
    """Name the case before each GPU step (flushed, so a crash still shows it)."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def dev(a: np.ndarray):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def row_rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max over rows (all axes but the last) of max|o-r| / max|r|."""
    out = out.astype(np.float64).reshape(-1, out.shape[-1])
    ref = ref.astype(np.float64).reshape(-1, ref.shape[-1])
    den = np.abs(ref).max(axis=1)
    num = np.abs(out - ref).max(axis=1)
    ok = den > 0
    worst = float((num[ok] / den[ok]).max()) if ok.any() else 0.0
    if (~ok).any():   # rows whose reference is exactly zero must be exactly zero
        worst = max(worst, float(num[~ok].max()) * 1e30)
    return worst


def vt_position(k: np.ndarray) -> np.ndarray:
    """Position of key k in a feature row of the dense path's fp16 value form
    (include/dsa.h, dsa_dense_masked_attn_f16): 32 (k / 32) + vt_pos(k % 32)."""
    x = k % 32
    return 32 * (k // 32) + 8 * ((x % 16) // 4) + 4 * (x // 16) + x % 4


def vt_layout(vals: np.ndarray, Np: int) -> np.ndarray:
    """[N, H, Dv] 16-bit patterns -> the [H, Dv, Np] value form, zeros past N."""
    N, H, Dv = vals.shape
    out = np.zeros((H, Dv, Np), dtype=vals.dtype)
    out[:, :, vt_position(np.arange(N))] = np.transpose(vals, (1, 2, 0))
    return out

