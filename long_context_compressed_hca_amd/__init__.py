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
        L.hca_decode_workspace_size.argtypes = [I, I, I, I64]
        L.hca_decode_workspace_size.restype = ctypes.c_size_t
        L.hca_attn_decode.argtypes = [P, P, P, P, I64, P, P, P, I, I, I, I, I, F, P, I, P,
                                      ctypes.c_size_t, P]
        L.hca_attn_decode.restype = I
        L.hca_attn_decode_noalloc.argtypes = [P, P, P, P, I64, P, P, P, I, I, I, I, I, F, P, I, P]
        L.hca_attn_decode_noalloc.restype = I
        L.hca_gate_logits.argtypes = [P, P, I64, I, I, P, P]
        L.hca_gate_logits.restype = I
        L.hca_attn_decode_multi.argtypes = [P, P, P, P, I64, P, P, P, P, P, I, I, I, I, I, I, F,
                                            P, I, P]
        L.hca_attn_decode_multi.restype = I
        L.hca_attn_prefill_vha.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, I, I, I, I,
                                           F, P, P, I, P, I, P]
        L.hca_attn_prefill_vha.restype = I
        L.hca_backward_workspace_size.argtypes = [I64, I, I]
        L.hca_backward_workspace_size.restype = ctypes.c_size_t
        L.hca_attn_backward.argtypes = [P, P, P, P, P, P, P, I64, I, I, I, I, F, P, P, P, P, P,
                                        ctypes.c_size_t, P]
        L.hca_attn_backward.restype = I
        L.hca_attn_prefill_lse.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, I, I, I, I,
                                           F, P, I, P, P]
        L.hca_attn_prefill_lse.restype = I
        L.hca_attn_backward_saved.argtypes = [P, P, P, P, P, P, P, I, P, P, I64, I, I, I, I, F, P,
                                              P, P, P, P, ctypes.c_size_t, P]
        L.hca_attn_backward_saved.restype = I
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


def _expect(t, shape, name):
    """Raise ValueError unless tensor t (or None) has exactly `shape`."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(map(str, devs))}")


def _stream(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def hca_compress(k, v, ck, cv, *, block: int = BLOCK):
    """ck, cv [T // 128, 512] <- block means of k, v [T, 512] (bf16).  k/ck or v/cv may be None."""
    import torch
    ref = k if k is not None else v
    if ref is None:
        raise ValueError("k and v are both None")
    if ref.dim() != 2:
        raise ValueError("k and v must be [T, D]")
    T, Dd = ref.shape
    for x, c, n in ((k, ck, "k"), (v, cv, "v")):
        if (x is None) != (c is None):
            raise ValueError(f"{n} and c{n} must be both given or both None")
        _expect(x, (T, Dd), n)
        _expect(c, (T // block, Dd), "c" + n)
    _same_device(k, v, ck, cv)
    _check(lib().hca_compress(_dev_ptr(k, "k", torch.bfloat16, True),
                              _dev_ptr(v, "v", torch.bfloat16, True), T, Dd, Dd, block,
                              _dev_ptr(ck, "ck", torch.bfloat16, True),
                              _dev_ptr(cv, "cv", torch.bfloat16, True), _stream(ref.device)))


def _check_prefill_shapes(q, g, k, v, ck, cv, out) -> int:
    """Shape checks shared by the prefill entry points; returns Nc."""
    import torch
    if q.dim() != 3:
        raise ValueError("q must be [Tq, H, D]")
    Dd = q.shape[2]
    _expect(g, q.shape, "g")
    _expect(out, q.shape, "out")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    if k.dim() != 2 or k.shape[1] != Dd:
        raise ValueError(f"k must be [Tkv, {Dd}], got {tuple(k.shape)}")
    _expect(v, k.shape, "v")
    if (ck is None) != (cv is None):
        raise ValueError("ck and cv must be both given or both None")
    nc = 0
    if ck is not None:
        if ck.dim() != 2 or ck.shape[1] != Dd:
            raise ValueError(f"ck must be [Nc, {Dd}], got {tuple(ck.shape)}")
        _expect(cv, ck.shape, "cv")
        nc = ck.shape[0]
    _same_device(q, g, k, v, ck, cv, out)
    return nc


def hca_attn_prefill(q, g, k, v, ck, cv, out, *, q_start: int = 0, kv_start: int = 0,
                     scale: float | None = None, block: int = BLOCK, window: int = WINDOW):
    """out [Tq, H, 512] <- HCA attention of queries at q_start.. over entries ck/cv and raw
    rows k/v starting at position kv_start, gated by sigmoid(g)."""
    import torch
    Tq, H, Dd = q.shape
    nc = _check_prefill_shapes(q, g, k, v, ck, cv, out)
    if scale is None:
        scale = Dd ** -0.5
    _check(lib().hca_attn_prefill(
        _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(g, "g", torch.bfloat16),
        _dev_ptr(k, "k", torch.bfloat16), _dev_ptr(v, "v", torch.bfloat16),
        _dev_ptr(ck, "ck", torch.bfloat16, True), _dev_ptr(cv, "cv", torch.bfloat16, True),
        Tq, q_start, k.shape[0], kv_start, nc, H, Dd, block, window, float(scale),
        _dev_ptr(out, "out"), HCA_F32 if out.dtype == torch.float32 else HCA_BF16,
        _stream(q.device)))


def hca_attn_prefill_lse(q, g, k, v, ck, cv, out, lse, *, q_start: int = 0, kv_start: int = 0,
                         scale: float | None = None, block: int = BLOCK, window: int = WINDOW):
    """hca_attn_prefill, and lse [Tq, H] (float32) <- each row's log-sum-exp of its
    scores (natural log), the state hca_attn_backward_saved takes."""
    import torch
    Tq, H, Dd = q.shape
    nc = _check_prefill_shapes(q, g, k, v, ck, cv, out)
    _expect(lse, (Tq, H), "lse")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    _same_device(q, lse)
    if scale is None:
        scale = Dd ** -0.5
    _check(lib().hca_attn_prefill_lse(
        _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(g, "g", torch.bfloat16),
        _dev_ptr(k, "k", torch.bfloat16), _dev_ptr(v, "v", torch.bfloat16),
        _dev_ptr(ck, "ck", torch.bfloat16, True), _dev_ptr(cv, "cv", torch.bfloat16, True),
        Tq, q_start, k.shape[0], kv_start, nc, H, Dd, block, window, float(scale),
        _dev_ptr(out, "out"), HCA_F32 if out.dtype == torch.float32 else HCA_BF16,
        _dev_ptr(lse, "lse", torch.float32), _stream(q.device)))


def _check_cache_shapes(B, Dd, ck, cv, wk, wv, pos, window) -> int:
    """Shape checks of a decode call's per-sequence cache; returns nc_cap."""
    if (ck is None) != (cv is None):
        raise ValueError("ck and cv must be both given or both None")
    nc_cap = 0
    if ck is not None:
        if ck.dim() != 3 or ck.shape[0] != B or ck.shape[2] != Dd:
            raise ValueError(f"ck must be [{B}, nc_cap, {Dd}], got {tuple(ck.shape)}")
        _expect(cv, ck.shape, "cv")
        nc_cap = ck.shape[1]
    _expect(wk, (B, window, Dd), "wk")
    _expect(wv, (B, window, Dd), "wv")
    _expect(pos, (B,), "pos")
    return nc_cap


def decode_workspace_size(B: int, H: int, nc_cap: int, D: int = D) -> int:
    """Bytes of device workspace hca_attn_decode needs (0: none)."""
    return int(lib().hca_decode_workspace_size(B, H, D, nc_cap))


def hca_attn_decode(q, g, ck, cv, wk, wv, pos, out, *, scale: float | None = None,
                    workspace=None, block: int = BLOCK, window: int = WINDOW):
    """out [B, H, 512] <- HCA decode for one new token per sequence at positions pos [B]
    (int64, on the GPU), with per-sequence entries ck/cv [B, nc_cap, 512] and rings
    wk/wv [B, 128, 512] (position p in slot p % 128).  workspace: a device uint8 tensor
    of at least decode_workspace_size(B, H, nc_cap) bytes; allocated here (through
    torch) when None and needed."""
    import torch
    if q.dim() != 3:
        raise ValueError("q must be [B, H, D]")
    B, H, Dd = q.shape
    _expect(g, q.shape, "g")
    _expect(out, q.shape, "out")
    nc_cap = _check_cache_shapes(B, Dd, ck, cv, wk, wv, pos, window)
    _same_device(q, g, ck, cv, wk, wv, pos, out)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    if scale is None:
        scale = Dd ** -0.5
    need = decode_workspace_size(B, H, nc_cap, Dd) if B > 0 else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hca_attn_decode(
        _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(g, "g", torch.bfloat16),
        _dev_ptr(ck, "ck", torch.bfloat16, True), _dev_ptr(cv, "cv", torch.bfloat16, True),
        nc_cap, _dev_ptr(wk, "wk", torch.bfloat16), _dev_ptr(wv, "wv", torch.bfloat16),
        _dev_ptr(pos, "pos", torch.int64), B, H, Dd, block, window, float(scale),
        _dev_ptr(out, "out"), HCA_F32 if out.dtype == torch.float32 else HCA_BF16,
        _dev_ptr(workspace, "workspace", optional=True), ws_bytes, _stream(q.device)))


def hca_attn_decode_noalloc(q, g, ck, cv, wk, wv, pos, out, *, scale: float | None = None,
                            block: int = BLOCK, window: int = WINDOW):
    """hca_attn_decode without a workspace argument: split batches use the library's
    built-in per-GPU scratch, so the call allocates nothing.  Calls overlapping on one
    GPU race on that scratch."""
    import torch
    if q.dim() != 3:
        raise ValueError("q must be [B, H, D]")
    B, H, Dd = q.shape
    _expect(g, q.shape, "g")
    _expect(out, q.shape, "out")
    nc_cap = _check_cache_shapes(B, Dd, ck, cv, wk, wv, pos, window)
    _same_device(q, g, ck, cv, wk, wv, pos, out)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    if scale is None:
        scale = Dd ** -0.5
    _check(lib().hca_attn_decode_noalloc(
        _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(g, "g", torch.bfloat16),
        _dev_ptr(ck, "ck", torch.bfloat16, True), _dev_ptr(cv, "cv", torch.bfloat16, True),
        nc_cap, _dev_ptr(wk, "wk", torch.bfloat16), _dev_ptr(wv, "wv", torch.bfloat16),
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
    if q.dim() != 4:
        raise ValueError("q must be [B, M, H, D]")
    B, M, H, Dd = q.shape
    _expect(g, q.shape, "g")
    _expect(out, q.shape, "out")
    _expect(nk, (B, M, Dd), "nk")
    _expect(nv, (B, M, Dd), "nv")
    nc_cap = _check_cache_shapes(B, Dd, ck, cv, wk, wv, pos, window)
    _same_device(q, g, ck, cv, wk, wv, nk, nv, pos, out)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    if scale is None:
        scale = Dd ** -0.5
    _check(lib().hca_attn_decode_multi(
        _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(g, "g", torch.bfloat16),
        _dev_ptr(ck, "ck", torch.bfloat16, True), _dev_ptr(cv, "cv", torch.bfloat16, True),
        nc_cap, _dev_ptr(wk, "wk", torch.bfloat16), _dev_ptr(wv, "wv", torch.bfloat16),
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
    nc = _check_prefill_shapes(q, g, k, v, ck, cv, out)
    if up.dim() != 2:
        raise ValueError("up must be [H, r]")
    r = up.shape[1]
    if up.shape != (H, r) or down.shape != (r, H):
        raise ValueError("up must be [H, r] and down [r, H]")
    _same_device(q, up, down)
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


def hca_gate_logits(latent, w_g, g):
    """g [T, N] (or [T, H, 512] with N = H * 512) <- bf16(latent [T, R] @ w_g [N, R]^T):
    the logits of the low-rank gate."""
    import torch
    if latent.dim() != 2 or w_g.dim() != 2 or w_g.shape[1] != latent.shape[1]:
        raise ValueError("latent must be [T, R] and w_g [N, R]")
    T, R = latent.shape
    N = w_g.shape[0]
    if g.numel() != T * N or g.shape[0] != T:
        raise ValueError(f"g must hold [{T}, {N}]")
    _same_device(latent, w_g, g)
    _check(lib().hca_gate_logits(_dev_ptr(latent, "latent", torch.bfloat16),
                                 _dev_ptr(w_g, "w_g", torch.bfloat16), T, R, N,
                                 _dev_ptr(g, "g", torch.bfloat16), _stream(latent.device)))


def hca_attn_prefill_lowrank_gate(q, latent, w_g, k, v, ck, cv, out, *, g=None, q_start: int = 0,
                                  kv_start: int = 0, scale: float | None = None):
    """HCA prefill gated by the low-rank gate: g = latent @ w_g^T (hca_gate_logits, into
    ``g`` or a buffer allocated here) followed by hca_attn_prefill on it."""
    import torch
    Tq, H, Dd = q.shape
    if g is None:
        g = torch.empty((Tq, H, Dd), dtype=torch.bfloat16, device=q.device)
    hca_gate_logits(latent, w_g, g)
    hca_attn_prefill(q, g, k, v, ck, cv, out, q_start=q_start, kv_start=kv_start, scale=scale)
    return g


def backward_workspace_size(T: int, H: int, D: int = D) -> int:
    """Bytes of device workspace hca_attn_backward needs (0 for T = 0 or an
    unsupported shape)."""
    return int(lib().hca_backward_workspace_size(T, H, D))


def hca_attn_backward(q, g, k, v, ck, cv, dout, dq, dk, dv, dg, *, scale: float | None = None,
                      workspace=None, block: int = BLOCK, window: int = WINDOW):
    """Gradients of a whole-sequence HCA prefill (queries and raw rows at positions
    0 .. T-1, ck/cv the floor(T/128) entries of k/v) for the upstream gradient dout of
    the gated output: dq, dg [T, H, 512] and dk, dv [T, 512], float32, overwritten.
    An entry's gradient reaches each raw row of its block divided by 128.  workspace:
    a device uint8 tensor of at least backward_workspace_size(T, H) bytes; allocated
    here (through torch) when None."""
    import torch
    T, H, Dd, scale, workspace, ws_bytes = _backward_args(q, g, k, v, ck, cv, dout, dq, dk, dv,
                                                          dg, scale, workspace, block)
    _check(lib().hca_attn_backward(
        _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(g, "g", torch.bfloat16),
        _dev_ptr(k, "k", torch.bfloat16), _dev_ptr(v, "v", torch.bfloat16),
        _dev_ptr(ck, "ck", torch.bfloat16, True), _dev_ptr(cv, "cv", torch.bfloat16, True),
        _dev_ptr(dout, "dout", torch.bfloat16), T, H, Dd, block, window, float(scale),
        _dev_ptr(dq, "dq", torch.float32), _dev_ptr(dk, "dk", torch.float32),
        _dev_ptr(dv, "dv", torch.float32), _dev_ptr(dg, "dg", torch.float32),
        _dev_ptr(workspace, "workspace", optional=True), ws_bytes, _stream(q.device)))


def hca_attn_backward_saved(q, g, k, v, ck, cv, out, lse, dout, dq, dk, dv, dg, *,
                            scale: float | None = None, workspace=None, block: int = BLOCK,
                            window: int = WINDOW):
    """hca_attn_backward from the forward's saved state: its gated output out [T, H, 512]
    (bfloat16 or float32) and row log-sum-exp lse [T, H] (float32), as
    hca_attn_prefill_lse writes them."""
    import torch
    T, H, Dd, scale, workspace, ws_bytes = _backward_args(q, g, k, v, ck, cv, dout, dq, dk, dv,
                                                          dg, scale, workspace, block)
    _expect(out, q.shape, "out")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    _expect(lse, (T, H), "lse")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    _same_device(q, out, lse)
    _check(lib().hca_attn_backward_saved(
        _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(g, "g", torch.bfloat16),
        _dev_ptr(k, "k", torch.bfloat16), _dev_ptr(v, "v", torch.bfloat16),
        _dev_ptr(ck, "ck", torch.bfloat16, True), _dev_ptr(cv, "cv", torch.bfloat16, True),
        _dev_ptr(out, "out"), HCA_F32 if out.dtype == torch.float32 else HCA_BF16,
        _dev_ptr(lse, "lse", torch.float32), _dev_ptr(dout, "dout", torch.bfloat16), T, H, Dd,
        block, window, float(scale), _dev_ptr(dq, "dq", torch.float32),
        _dev_ptr(dk, "dk", torch.float32), _dev_ptr(dv, "dv", torch.float32),
        _dev_ptr(dg, "dg", torch.float32), _dev_ptr(workspace, "workspace", optional=True),
        ws_bytes, _stream(q.device)))


def _backward_args(q, g, k, v, ck, cv, dout, dq, dk, dv, dg, scale, workspace, block):
    """Shape, dtype and device checks shared by the backward entry points; returns
    (T, H, D, scale, workspace, ws_bytes) with the workspace allocated if None."""
    import torch
    if q.dim() != 3:
        raise ValueError("q must be [T, H, D]")
    T, H, Dd = q.shape
    for t, name in ((g, "g"), (dout, "dout")):
        _expect(t, q.shape, name)
    for t, name in ((dq, "dq"), (dg, "dg")):
        _expect(t, q.shape, name)
    for t, name in ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")):
        _expect(t, (T, Dd), name)
    Nc = T // block
    for t, name in ((ck, "ck"), (cv, "cv")):
        if t is not None:
            _expect(t, (t.shape[0], Dd), name)
            if t.shape[0] < Nc:
                raise ValueError(f"{name} holds {t.shape[0]} entries, {Nc} needed")
        elif Nc > 0:
            raise ValueError(f"{name} is needed for T >= {block}")
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv"), (dg, "dg")):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    _same_device(*(t for t in (q, g, k, v, ck, cv, dout, dq, dk, dv, dg) if t is not None))
    if scale is None:
        scale = Dd ** -0.5
    need = backward_workspace_size(T, H, Dd) if T > 0 else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return T, H, Dd, scale, workspace, ws_bytes
