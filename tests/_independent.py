"""Independent test-only computations that pin the oracle.

None of these call the oracle.  Each computes the same quantity by a different
route: dense matrix algebra with an explicit boolean mask (numpy BLAS), exact
rational arithmetic (fractions), or a library attention routine (torch SDPA).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def widen(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def dense_masked_attention(q, g, tpos, k, v, kv_start, ck, cv, block, window, scale):
    """Brute force: one dense key matrix [raw rows; compressed entries], a
    boolean visibility matrix built from the two rules, softmax with -inf on
    hidden keys, then the sigmoid gate.  float64 throughout."""
    qf, gf = widen(q), widen(g)
    kaug = np.concatenate([widen(k), widen(ck)], axis=0)
    vaug = np.concatenate([widen(v), widen(cv)], axis=0)
    raw_pos = kv_start + np.arange(k.shape[0])
    block_last = np.arange(ck.shape[0]) * block + (block - 1)
    t = np.asarray(tpos, dtype=np.int64)[:, None]
    visible = np.concatenate([(raw_pos[None, :] <= t) & (raw_pos[None, :] > t - window),
                              block_last[None, :] <= t], axis=1)          # [n, keys]
    s = scale * np.einsum("nhd,jd->nhj", qf, kaug)
    s = np.where(visible[:, None, :], s, -np.inf)
    s = s - s.max(axis=2, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=2, keepdims=True)
    o = np.einsum("nhj,jd->nhd", p, vaug)
    return o / (1.0 + np.exp(-gf))


def exact_bf16_round(x: Fraction) -> Fraction:
    """Round a rational to the nearest bfloat16 value, ties to even (exact)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = 0                      # find e with 2^e <= a < 2^(e+1)
    while a >= Fraction(2) ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    qexp = max(e - 7, -133)    # 8 significant bits; subnormal quantum 2^-133
    quantum = Fraction(2) ** qexp
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def exact_block_mean_bf16(x_bits, block):
    """Compressed entries by exact rational mean + exact RNE; returns Fractions [nb][D]."""
    x = widen(x_bits)
    T, D = x.shape
    out = []
    for b in range(T // block):
        row = []
        for d in range(D):
            s = sum(Fraction(float(x[b * block + i, d])) for i in range(block))
            row.append(exact_bf16_round(s / block))
        out.append(row)
    return out


def sdpa_causal(q, g, k, v, scale):
    """T <= window-1 and no completed block: HCA is plain causal attention with one
    shared K/V head.  Uses torch's scaled_dot_product_attention in float64."""
    import torch
    qf = torch.from_numpy(widen(q)).permute(1, 0, 2)            # [H, T, D]
    H = qf.shape[0]
    kf = torch.from_numpy(widen(k))[None].expand(H, -1, -1).contiguous()
    vf = torch.from_numpy(widen(v))[None].expand(H, -1, -1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qf, kf, vf, is_causal=True, scale=scale)
    gate = torch.sigmoid(torch.from_numpy(widen(g)).permute(1, 0, 2))
    return (o * gate).permute(1, 0, 2).numpy()


def dense_attention_f64(qf, gf, kf, vf, block, window, scale):
    """The layer's forward pass from float64 arrays with no rounding anywhere
    (entries are the exact block means of kf, vf): a dense key matrix, a boolean
    visibility matrix, softmax, values, sigmoid gate.  Used for finite
    differences and as the autograd graph for the backward pins."""
    T, H, D = qf.shape
    nc = T // block
    ckf = kf[:nc * block].reshape(nc, block, D).mean(axis=1)
    cvf = vf[:nc * block].reshape(nc, block, D).mean(axis=1)
    kaug = np.concatenate([kf, ckf], axis=0)
    vaug = np.concatenate([vf, cvf], axis=0)
    pos = np.arange(T)
    block_last = np.arange(nc) * block + (block - 1)
    t = pos[:, None]
    visible = np.concatenate([(pos[None, :] <= t) & (pos[None, :] > t - window),
                              block_last[None, :] <= t], axis=1)
    s = scale * np.einsum("thd,jd->thj", qf, kaug)
    s = np.where(visible[:, None, :], s, -np.inf)
    s = s - s.max(axis=2, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=2, keepdims=True)
    return np.einsum("thj,jd->thd", p, vaug) / (1.0 + np.exp(-gf))
