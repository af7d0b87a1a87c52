"""ctypes front end of the fp64 HCA oracle in ``hca_oracle.c``.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark are the only users.  Nothing in the HIP library imports,
links or calls this package, and this package imports nothing from the HIP
library.  Arrays of bfloat16 values travel as ``numpy.uint16`` bit patterns.

What each function computes is documented at its C definition, with the page
and section it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hca_oracle.c")
LIB = os.path.join(HERE, "libhca_oracle.so")

_lib = None


def build() -> str:
    """Compile the oracle with gcc (plain IEEE double, no FMA contraction)."""
    tmp = LIB + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
         "-fno-fast-math", "-Wall", "-Wextra", SRC, "-o", tmp, "-lm"])
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    _lib = bind(ctypes.CDLL(LIB))
    return _lib


def bind(lib):
    """Declare the C signatures on a loaded oracle library."""
    P, I64, I, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.hca_oracle_compress.argtypes = [P, I64, I64, I, I, P]
    lib.hca_oracle_attn.argtypes = [P, P, P, I64, P, P, I64, I64, P, P, I64, I, I, I, I, D, P, I]
    lib.hca_oracle_decode.argtypes = [P, P, P, P, I64, P, P, P, I, I, I, I, I, D, P, I]
    lib.hca_oracle_attn_backward.argtypes = [P, P, P, I64, P, P, P, P, I64, I, I, I, I, D, P, P,
                                             P, P, P, P, I]
    lib.hca_oracle_attn_backward_rows.argtypes = [P, P, P, P, I64, I64, P, P, P, P, I64, I, I, I,
                                                  I, D, P, P, I]
    lib.hca_oracle_attn_lse.argtypes = [P, P, I64, P, I64, I64, P, I64, I, I, I, I, D, P, I]
    lib.hca_oracle_attn_backward_saved.argtypes = [P, P, P, P, P, I64, P, P, P, P, I64, I, I, I,
                                                   I, D, I, P, P, P, P, P, P, I]
    lib.hca_oracle_round_bf16.argtypes = [D]
    lib.hca_oracle_round_bf16.restype = ctypes.c_uint16
    lib.hca_oracle_widen_bf16.argtypes = [ctypes.c_uint16]
    lib.hca_oracle_widen_bf16.restype = D
    lib.hca_oracle_threads.restype = I
    return lib


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bfloat16 data travels as uint16 bit patterns")
    return a


def threads() -> int:
    return _load().hca_oracle_threads()


def round_bf16(x: float) -> int:
    return int(_load().hca_oracle_round_bf16(float(x)))


def widen_bf16(bits: int) -> float:
    return float(_load().hca_oracle_widen_bf16(int(bits)))


def compress(x, block: int = 128) -> np.ndarray:
    """Mean of each complete ``block`` of rows of ``x`` [T, D], rounded to bf16."""
    x = _u16(x)
    T, D = x.shape
    out = np.zeros((T // block, D), dtype=np.uint16)
    rc = _load().hca_oracle_compress(_ptr(x), T, D, D, block, _ptr(out))
    if rc:
        raise OracleError(f"hca_oracle_compress: {rc}")
    return out


def attn(q, g, tpos, k, v, kv_start, ck, cv, *, block=128, window=128, scale=None,
         nthreads=0) -> np.ndarray:
    """HCA attention rows.  q, g: [n, H, D]; tpos: [n] positions; k, v: raw rows
    from ``kv_start``; ck, cv: [Nc, D] entries.  Returns float64 [n, H, D]."""
    q, g, k, v = _u16(q), _u16(g), _u16(k), _u16(v)
    ck = _u16(ck) if ck is not None else np.zeros((0, q.shape[2]), np.uint16)
    cv = _u16(cv) if cv is not None else np.zeros((0, q.shape[2]), np.uint16)
    n, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    tpos = np.ascontiguousarray(tpos, dtype=np.int64)
    assert tpos.shape == (n,) and g.shape == q.shape
    out = np.empty((n, H, D), dtype=np.float64)
    rc = _load().hca_oracle_attn(_ptr(q), _ptr(g), _ptr(tpos), n, _ptr(k), _ptr(v), k.shape[0],
                                 int(kv_start), _ptr(ck), _ptr(cv), ck.shape[0], H, D, block,
                                 window, float(scale), _ptr(out), int(nthreads))
    if rc:
        raise OracleError(f"hca_oracle_attn: {rc}")
    return out


def decode(q, g, ck, cv, wk, wv, pos, *, block=128, window=128, scale=None,
           nthreads=0) -> np.ndarray:
    """Decode rows.  q, g: [B, H, D]; ck, cv: [B, nc_cap, D]; wk, wv: [B, window, D]
    rings (position p in slot p % window); pos: [B].  Returns float64 [B, H, D]."""
    q, g, wk, wv = _u16(q), _u16(g), _u16(wk), _u16(wv)
    ck, cv = _u16(ck), _u16(cv)
    B, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    assert pos.shape == (B,) and wk.shape == (B, window, D)
    out = np.empty((B, H, D), dtype=np.float64)
    rc = _load().hca_oracle_decode(_ptr(q), _ptr(g), _ptr(ck), _ptr(cv), ck.shape[1], _ptr(wk),
                                   _ptr(wv), _ptr(pos), B, H, D, block, window, float(scale),
                                   _ptr(out), int(nthreads))
    if rc:
        raise OracleError(f"hca_oracle_decode: {rc}")
    return out


def decode_multi(q, g, ck, cv, wk, wv, nk, nv, pos, *, block=128, window=128, scale=None,
                 nthreads=0) -> np.ndarray:
    """Multi-token decode: M new tokens per sequence at positions pos .. pos+M-1, as
    when a drafter's tokens are verified in one pass (the ECHO layer doubles as a
    speculative-decoding drafter: blog.derekhsu.net, section "ECHO：取代 MTP 模組";
    two-step drafts in low-latency serving: lininn.cn, section "把 MTP 模块删了").
    Each new token is an ordinary query at its own
    position, so it attends to the entries of the blocks completed at or before it,
    to the committed raw rows of its window, and to the new tokens up to itself.

      q, g    [B, M, H, D]        queries and gate logits of the new tokens
      ck, cv  [B, nc_cap, D]      entries (the first floor((pos+M)/block) are used)
      wk, wv  [B, window, D]      ring of committed rows: position p < pos in slot p % window
      nk, nv  [B, M, D]           raw rows of the new tokens (positions pos .. pos+M-1)
      pos     [B]                 position of the first new token

    Composed from ``attn``: per sequence the raw rows max(0, pos-window+1) .. pos-1 are
    taken from the ring, followed by the M new rows, and ``attn`` is called with the
    queries at positions pos .. pos+M-1.  Returns float64 [B, M, H, D]."""
    q, g, wk, wv, nk, nv = _u16(q), _u16(g), _u16(wk), _u16(wv), _u16(nk), _u16(nv)
    ck, cv = _u16(ck), _u16(cv)
    B, M, H, D = q.shape
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    assert pos.shape == (B,) and nk.shape == (B, M, D) and wk.shape == (B, window, D)
    out = np.empty((B, M, H, D), dtype=np.float64)
    for b in range(B):
        t = int(pos[b])
        if t < 0 or (t + M) // block > ck.shape[1]:
            raise OracleError("decode_multi: position out of range")
        lo = max(0, t - window + 1)
        slots = [p % window for p in range(lo, t)]
        k = np.concatenate([wk[b, slots], nk[b]]) if slots else nk[b]
        v = np.concatenate([wv[b, slots], nv[b]]) if slots else nv[b]
        nc = (t + M) // block
        out[b] = attn(q[b], g[b], t + np.arange(M), k, v, lo, ck[b, :nc], cv[b, :nc],
                      block=block, window=window, scale=scale, nthreads=nthreads)
    return out


def vha(x, up, down) -> np.ndarray:
    """Virtual head attention: after attention, a low-rank mix across heads with an
    identity skip (blog.derekhsu.net, section 潛在閘控稀疏注意力, the VHA item).
    For every position t and dim d the head vector x[t, :, d] becomes
        y[t, h, d] = x[t, h, d] + sum_k up[h, k] * z[t, k, d],
        z[t, k, d] = sum_h' down[k, h'] * x[t, h', d],
    i.e. y = (I + up @ down) x over the heads, the same mix for every dim.
      x     [T, H, D]  float64 (the gated attention output)
      up    [H, r]     bfloat16 bits
      down  [r, H]     bfloat16 bits
    Returns float64 [T, H, D]."""
    x = np.asarray(x, dtype=np.float64)
    U, W = _widen_array(up), _widen_array(down)
    T, H, D = x.shape
    assert U.shape[0] == H and W.shape == (U.shape[1], H)
    z = np.einsum("kh,thd->tkd", W, x)
    return x + np.einsum("hk,tkd->thd", U, z)


def _widen_array(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64, exactly (the bits are the top half of a float32)."""
    b = _u16(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def attn_vha(q, g, tpos, k, v, kv_start, ck, cv, up, down, **kw) -> np.ndarray:
    """HCA attention rows (``attn``), gated, then the VHA head mix (``vha``)."""
    return vha(attn(q, g, tpos, k, v, kv_start, ck, cv, **kw), up, down)


def gate_logits(latent, w_g) -> np.ndarray:
    """Gate logits of the low-rank gate: the gate is computed from the query's
    low-rank latent, several times narrower than the hidden state
    (blog.derekhsu.net, section 潛在閘控稀疏注意力, the 低秩閘控注意力 item;
    yilup.net, section 架構設計: far fewer gate weights than a full-width gate).
        G[t, n] = sum_r latent[t, r] * W_g[n, r]
    with n = h * D + d indexing (head, dim) of the gate, i.e. G = latent @ W_g^T.
      latent  [T, R]   bfloat16 bits (R = 1024: 4096 hidden / 4)
      w_g     [N, R]   bfloat16 bits, out x in like a linear layer's weight (N = H * D)
    Returns float64 [T, N] (no rounding)."""
    return _widen_array(latent) @ _widen_array(w_g).T


def attn_lowrank_gate(q, latent, w_g, tpos, k, v, kv_start, ck, cv, **kw) -> np.ndarray:
    """HCA attention rows gated by sigmoid of the low-rank gate logits: the
    ungated attention (``attn`` with G = +inf, whose sigmoid is exactly 1) times
    1 / (1 + exp(-G)), G = ``gate_logits(latent, w_g)`` reshaped to [n, H, D]
    (unrounded).  Returns float64 [n, H, D]."""
    q = _u16(q)
    n, H, D = q.shape
    ungated = attn(q, np.full(q.shape, 0x7F80, np.uint16), tpos, k, v, kv_start, ck, cv, **kw)
    G = gate_logits(latent, w_g).reshape(n, H, D)
    return ungated / (1.0 + np.exp(-G))


def attn_backward(q, g, dout, k, v, *, block=128, window=128, scale=None, nthreads=0):
    """Gradients of a whole-sequence prefill (queries and raw rows at positions
    0 .. T-1, entries = ``compress`` of k and v) for the upstream gradient dout
    of the gated output (the training pass; blog.derekhsu.net, section 訓練基礎設施).
    The attention part follows the chain rule row by row (C routine
    ``hca_oracle_attn_backward``); then each entry's gradient reaches every raw row
    of its block divided by the block size, the derivative of the mean (the
    bfloat16 rounding of an entry is passed through as the identity).
      q, g, dout [T, H, D], k, v [T, D]: bfloat16 bits
    Returns float64 (dq [T, H, D], dk [T, D], dv [T, D], dg [T, H, D])."""
    q, g, dout, k, v = _u16(q), _u16(g), _u16(dout), _u16(k), _u16(v)
    T, H, D = q.shape
    assert g.shape == q.shape and dout.shape == q.shape and k.shape == (T, D) == v.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    ck, cv = compress(k, block), compress(v, block)
    Nc = ck.shape[0]
    dq = np.empty((T, H, D)); dg = np.empty((T, H, D))
    dk = np.empty((T, D)); dv = np.empty((T, D))
    dck = np.zeros((max(Nc, 1), D)); dcv = np.zeros((max(Nc, 1), D))
    rc = _load().hca_oracle_attn_backward(
        _ptr(q), _ptr(g), _ptr(dout), T, _ptr(k), _ptr(v), _ptr(ck) if Nc else None,
        _ptr(cv) if Nc else None, Nc, H, D, block, window, float(scale), _ptr(dq), _ptr(dg),
        _ptr(dk), _ptr(dv), _ptr(dck), _ptr(dcv), int(nthreads))
    if rc:
        raise OracleError(f"hca_oracle_attn_backward: {rc}")
    if Nc:
        dk[:Nc * block] += np.repeat(dck[:Nc] / block, block, axis=0)
        dv[:Nc * block] += np.repeat(dcv[:Nc] / block, block, axis=0)
    return dq, dk, dv, dg


def attn_backward_rows(q, g, dout, positions, k, v, *, block=128, window=128, scale=None,
                       nthreads=0):
    """dq and dg of the query rows at the given positions of a whole sequence whose raw
    rows are k, v [T, D] (entries = ``compress`` of them), by the same per-row routine
    as ``attn_backward`` (C ``hca_oracle_attn_backward_rows``); the key gradients need
    every row and are not formed.
      q, g, dout [n, H, D]: bfloat16 bits of the rows of positions[i]
    Returns float64 (dq [n, H, D], dg [n, H, D])."""
    q, g, dout, k, v = _u16(q), _u16(g), _u16(dout), _u16(k), _u16(v)
    n, H, D = q.shape
    T = k.shape[0]
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    assert g.shape == q.shape and dout.shape == q.shape and k.shape == (T, D) == v.shape
    assert pos.shape == (n,)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    ck, cv = compress(k, block), compress(v, block)
    Nc = ck.shape[0]
    dq = np.empty((n, H, D))
    dg = np.empty((n, H, D))
    rc = _load().hca_oracle_attn_backward_rows(
        _ptr(q), _ptr(g), _ptr(dout), _ptr(pos), n, T, _ptr(k), _ptr(v),
        _ptr(ck) if Nc else None, _ptr(cv) if Nc else None, Nc, H, D, block, window,
        float(scale), _ptr(dq), _ptr(dg), int(nthreads))
    if rc:
        raise OracleError(f"hca_oracle_attn_backward_rows: {rc}")
    return dq, dg



def attn_lse(q, tpos, k, kv_start, ck, *, block=128, window=128, scale=None, nthreads=0):
    """Per-row log-sum-exp of the scores, ln sum_j exp(scale <q, key_j>) over the keys
    each query sees (C ``hca_oracle_attn_lse``; the key list of ``attn``).
      q [n, H, D], k [Tkv, D] (positions kv_start ..), ck [Nc, D]: bfloat16 bits
    Returns float64 [n, H]."""
    q, k = _u16(q), _u16(k)
    n, H, D = q.shape
    tpos = np.ascontiguousarray(tpos, dtype=np.int64)
    assert tpos.shape == (n,) and k.shape[1] == D
    ck = None if ck is None or len(ck) == 0 else _u16(ck)
    Nc = 0 if ck is None else ck.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    lse = np.empty((n, H))
    rc = _load().hca_oracle_attn_lse(_ptr(q), _ptr(tpos), n, _ptr(k), k.shape[0], int(kv_start),
                                     _ptr(ck), Nc, H, D, block, window, float(scale), _ptr(lse),
                                     int(nthreads))
    if rc:
        raise OracleError(f"hca_oracle_attn_lse: {rc}")
    return lse


def attn_backward_saved(q, g, dout, out, lse, k, v, *, round_da=False, block=128, window=128,
                        scale=None, nthreads=0):
    """Gradients of a whole-sequence prefill from the forward's saved gated output
    ``out`` and row log-sum-exp ``lse`` (C ``hca_oracle_attn_backward_saved``: the
    weights come from lse, D = <dout, out>); entry gradients pooled to their raw
    rows as in ``attn_backward``.  With the exact out and lse and round_da off this
    equals ``attn_backward``; round_da rounds dA = dout * sigmoid(g) to bfloat16.
      q, g, dout [T, H, D], k, v [T, D]: bfloat16 bits;  out [T, H, D], lse [T, H]: float
    Returns float64 (dq [T, H, D], dk [T, D], dv [T, D], dg [T, H, D])."""
    q, g, dout, k, v = _u16(q), _u16(g), _u16(dout), _u16(k), _u16(v)
    T, H, D = q.shape
    out = np.ascontiguousarray(out, dtype=np.float64)
    lse = np.ascontiguousarray(lse, dtype=np.float64)
    assert g.shape == q.shape == dout.shape == out.shape and lse.shape == (T, H)
    assert k.shape == (T, D) == v.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    ck, cv = compress(k, block), compress(v, block)
    Nc = ck.shape[0]
    dq = np.empty((T, H, D)); dg = np.empty((T, H, D))
    dk = np.empty((T, D)); dv = np.empty((T, D))
    dck = np.zeros((max(Nc, 1), D)); dcv = np.zeros((max(Nc, 1), D))
    rc = _load().hca_oracle_attn_backward_saved(
        _ptr(q), _ptr(g), _ptr(dout), _ptr(out), _ptr(lse), T, _ptr(k), _ptr(v),
        _ptr(ck) if Nc else None, _ptr(cv) if Nc else None, Nc, H, D, block, window,
        float(scale), int(bool(round_da)), _ptr(dq), _ptr(dg), _ptr(dk), _ptr(dv), _ptr(dck),
        _ptr(dcv), int(nthreads))
    if rc:
        raise OracleError(f"hca_oracle_attn_backward_saved: {rc}")
    if Nc:
        dk[:Nc * block] += np.repeat(dck[:Nc] / block, block, axis=0)
        dv[:Nc * block] += np.repeat(dcv[:Nc] / block, block, axis=0)
    return dq, dk, dv, dg
