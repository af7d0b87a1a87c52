"""HCA (Heavily Compressed Attention) for AMD Instinct MI355X.

Thin ctypes binding of ``libhca.so`` (the C ABI of ``include/hca.h``): the
functions below only check tensor metadata and pass pointers, sizes and the
current HIP stream.  Every step of the computation runs in the HIP kernels;
there is no fallback.  Importing this package does not need a GPU; calling the
compute functions does, and they raise if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhca.so")

HCA_OK, HCA_ERR_INVALID_ARG, HCA_ERR_UNSUPPORTED, HCA_ERR_WORKSPACE, HCA_ERR_HIP = range(5)
HCA_BF16, HCA_F32 = 0, 1
D, BLOCK, WINDOW = 512, 128, 128

_lib = None


class HcaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def lib():
    """The loaded libhca.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.hca_status_string.argtypes = [I]
        L.hca_status_string.restype = ctypes.c_char_p
        L.hca_last_error.restype = ctypes.c_char_p
        L.hca_version.restype = I
        L.hca_compress.argtypes = [P, P, I64, I64, I, I, P, P, P]
        L.hca_compress.restype = I
        L.hca_attn_prefill.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, I, I, I, I, F,
                                       P, I, P]
        L.hca_attn_prefill.restype = I
        L.hca_attn_decode.argtypes = [P, P, P, P, I64, P, P, P, I, I, I, I, I, F, P, I, P]
        L.hca_attn_decode.restype = I
        L.hca_attn_decode_multi.argtypes = [P, P, P, P, I64, P, P, P, P, P, I, I, I, I, I, I, F,
                                            P, I, P]
        L.hca_attn_decode_multi.restype = I
        L.hca_attn_prefill_vha.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, I, I, I, I,
                                           F, P, P, I, P, I, P]
        L.hca_attn_prefill_vha.restype = I
        _lib = L
    return _lib


def _check(status: int):
    if status != HCA_OK:
        L = lib()
        raise HcaError(status, L.hca_last_error().decode() or L.hca_status_string(status).decode())


def _dev_ptr(t, name, dtype=None, optional=False):
    import torch
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a torch tensor on a GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def hca_compress(k, v, ck, cv, *, block: int = BLOCK):
    """ck, cv [T // 128, 512] <- block means of k, v [T, 512] (bf16).  k/ck or v/cv may be None."""
    import torch
    ref = k if k is not None else v
    T, Dd = ref.shape
    _check(lib().hca_compress(_dev_ptr(k, "k", torch.bfloat16, True),
                              _dev_ptr(v, "v", torch.bfloat16, True), T, Dd, Dd, block,
                              _dev_ptr(ck, "ck", torch.bfloat16, True),
                              _dev_ptr(cv, "cv", torch.bfloat16, True), _stream(ref.device)))


def hca_attn_prefill(q, g, k, v, ck, cv, out, *, q_start: int = 0, kv_start: int = 0,
                     scale: float | None = None, block: int = BLOCK, window: int = WINDOW):
    """out [Tq, H, 512] <- HCA attention of queries at q_start.. over entries ck/cv and raw
    rows k/v starting at position kv_start, gated by sigmoid(g)."""
    import torch
    Tq, H, Dd = q.shape
    if g.shape != q.shape or out.shape != q.shape:
        raise ValueError("q, g and out must have the same shape")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    nc = 0 if ck is None else ck.shape[0]
    if scale is None:
        scale = Dd ** -0.5
    _check(lib().hca_attn_prefill(
        _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(g, "g", torch.bfloat16),
        _dev_ptr(k, "k", torch.bfloat16), _dev_ptr(v, "v", torch.bfloat16),
        _dev_ptr(ck, "ck", torch.bfloat16, True), _dev_ptr(cv, "cv", torch.bfloat16, True),
        Tq, q_start, k.shape[0], kv_start, nc, H, Dd, block, window, float(scale),
        _dev_ptr(out, "out"), HCA_F32 if out.dtype == torch.float32 else HCA_BF16,
        _stream(q.device)))


def hca_attn_decode(q, g, ck, cv, wk, wv, pos, out, *, scale: float | None = None,
                    block: int = BLOCK, window: int = WINDOW):
    """out [B, H, 512] <- HCA decode for one new token per sequence at positions pos [B]
    (int64, on the GPU), with per-sequence entries ck/cv [B, nc_cap, 512] and rings
    wk/wv [B, 128, 512] (position p in slot p % 128)."""
    import torch
    B, H, Dd = q.shape
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    if scale is None:
        scale = Dd ** -0.5
    _check(lib().hca_attn_decode(
        _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(g, "g", torch.bfloat16),
        _dev_ptr(ck, "ck", torch.bfloat16, True), _dev_ptr(cv, "cv", torch.bfloat16, True),
        ck.shape[1], _dev_ptr(wk, "wk", torch.bfloat16), _dev_ptr(wv, "wv", torch.bfloat16),
        _dev_ptr(pos, "pos", torch.int64), B, H, Dd, block, window, float(scale),
        _dev_ptr(out, "out"), HCA_F32 if out.dtype == torch.float32 else HCA_BF16,
        _stream(q.device)))


def hca_attn_decode_multi(q, g, ck, cv, wk, wv, nk, nv, pos, out, *, scale: float | None = None,
                          block: int = BLOCK, window: int = WINDOW):
    """out [B, M, H, 512] <- HCA decode for M new tokens per sequence at positions
    pos .. pos+M-1 (pos [B] int64 on the GPU), each attending causally to the earlier
    new tokens.  Entries ck/cv [B, nc_cap, 512]; rings wk/wv [B, 128, 512] of committed
    rows (position p < pos in slot p % 128); the new tokens' rows nk/nv [B, M, 512]."""
    import torch
    B, M, H, Dd = q.shape
    if g.shape != q.shape or out.shape != q.shape:
        raise ValueError("q, g and out must have the same shape")
    if nk.shape != (B, M, Dd) or nv.shape != (B, M, Dd):
        raise ValueError("nk and nv must be [B, M, D]")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    if scale is None:
        scale = Dd ** -0.5
    _check(lib().hca_attn_decode_multi(
        _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(g, "g", torch.bfloat16),
        _dev_ptr(ck, "ck", torch.bfloat16, True), _dev_ptr(cv, "cv", torch.bfloat16, True),
        ck.shape[1], _dev_ptr(wk, "wk", torch.bfloat16), _dev_ptr(wv, "wv", torch.bfloat16),
        _dev_ptr(nk, "nk", torch.bfloat16), _dev_ptr(nv, "nv", torch.bfloat16),
        _dev_ptr(pos, "pos", torch.int64), B, M, H, Dd, block, window, float(scale),
        _dev_ptr(out, "out"), HCA_F32 if out.dtype == torch.float32 else HCA_BF16,
        _stream(q.device)))


def hca_attn_prefill_vha(q, g, k, v, ck, cv, up, down, out, *, q_start: int = 0,
                         kv_start: int = 0, scale: float | None = None, block: int = BLOCK,
                         window: int = WINDOW):
    """hca_attn_prefill followed by the VHA head mix out = (I + up @ down) x over the 64
    heads of each query; up [64, r], down [r, 64] bf16 on the GPU, r in 4, 8, .., 32."""
    import torch
    Tq, H, Dd = q.shape
    if g.shape != q.shape or out.shape != q.shape:
        raise ValueError("q, g and out must have the same shape")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    r = up.shape[1]
    if up.shape != (H, r) or down.shape != (r, H):
        raise ValueError("up must be [H, r] and down [r, H]")
    nc = 0 if ck is None else ck.shape[0]
    if scale is None:
        scale = Dd ** -0.5
    _check(lib().hca_attn_prefill_vha(
        _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(g, "g", torch.bfloat16),
        _dev_ptr(k, "k", torch.bfloat16), _dev_ptr(v, "v", torch.bfloat16),
        _dev_ptr(ck, "ck", torch.bfloat16, True), _dev_ptr(cv, "cv", torch.bfloat16, True),
        Tq, q_start, k.shape[0], kv_start, nc, H, Dd, block, window, float(scale),
        _dev_ptr(up, "up", torch.bfloat16), _dev_ptr(down, "down", torch.bfloat16), r,
        _dev_ptr(out, "out"), HCA_F32 if out.dtype == torch.float32 else HCA_BF16,
        _stream(q.device)))
