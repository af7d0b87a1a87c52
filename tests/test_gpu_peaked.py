"""Peaked softmax on the GPU: rows whose largest score lies far above the
largest score of the first key tile they see.

The kernels weigh each key by 2^(x - m) with x the score in base-2 units and
m a per-row reference taken early in the key walk (the maximum of the first
tile that holds a visible key).  A key scoring more than 64 (base 2) above
that reference sends a kernel down its exact-maximum path: prefill and the
decode kernels rescale or rerun with the true row maximum.  With N(0,1) inputs
at scale 1/sqrt(512) that never happens, so these tests build queries that
point at one or two late window keys:

    q[t, h] = bf16(c * (k[a] + k[b]))     a, b among the last raw rows of row t

The score of such a key is about c * 512 / sqrt(512) = 22.6 c (natural units),
while a compressed entry scores about c * N(0, 2) (entries are independent of
k[a], k[b]).  With c = 3 the gap is about 68 - 14 = 54 > 64 / log2(e) = 44.4.
Every test asserts this on the host, in fp64 from the bf16 inputs, for the rows
it counts (max over the aligned keys minus max over every visible entry, the
first tile's maximum being at most the latter), and compares every output with
the oracle at the usual tolerance.  Only some heads are aimed, so the items and
workgroups hold a mix of peaked and ordinary rows.
"""
import numpy as np
import pytest
import torch

import long_context_compressed_hca_amd as hca
import oracle
import synth
from tests.gpu_util import D, Prefill, compare, dev, gen, host, host_f64

pytestmark = pytest.mark.gpu

C = 3.0
GAP = 64.0 / np.log2(np.e) + 1.0   # natural units, with a margin for fp32 scores
SCALE = 512 ** -0.5


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(
        torch.bfloat16)


def _aim(qrow_bits, ka, kb):
    """bf16 bits of c * (ka + kb) (fp32 sum, nearest-even)."""
    v = (C * (_f64(ka) + _f64(kb))).astype(np.float32)
    return synth.f32_to_bf16_bits(v)


def _gap(q_bits, aimed_keys, entries):
    """max over aimed keys minus max over entries, scale * <q, k> in fp64."""
    q = _f64(q_bits)
    s_aim = max(float(q @ _f64(k)) for k in aimed_keys) * SCALE
    s_ent = float((_f64(entries) @ q).max()) * SCALE
    return s_aim - s_ent


def _peaked_prefill(seed, Tq, H, q_start=0, out_dtype="bf16", heads=None):
    """A Prefill problem whose rows at t >= 128 aim heads `heads` at k[t-1], k[t-3].
    Returns the problem and the number of rows that pass the host check."""
    p = Prefill(seed=seed, Tq=Tq, H=H, q_start=q_start, out_dtype=out_dtype)
    heads = range(0, H, 2) if heads is None else heads
    qh, kh = host(p.q), host(p.k_all)
    ck = oracle.compress(kh[:p.Nc * 128])
    n_over = 0
    for i in range(Tq):
        t = q_start + i
        nc = (t + 1) // 128
        if nc == 0:
            continue
        for h in heads:
            qh[i, h] = _aim(qh[i, h], kh[t - 1], kh[t - 3])
            if _gap(qh[i, h], (kh[t - 1], kh[t - 3]), ck[:nc]) > GAP:
                n_over += 1
    p.q = _to_dev(qh)
    return p, n_over


@pytest.mark.parametrize("Tq,H,q_start,out_dtype", [
    (600, 8, 0, "f32"),
    (300, 64, 0, "bf16"),
    (257, 64, 900, "f32"),
    (200, 3, 130, "bf16"),
])
def test_prefill_peaked_rows(Tq, H, q_start, out_dtype):
    p, n_over = _peaked_prefill(80 + H, Tq, H, q_start, out_dtype)
    rows = (Tq - max(0, 127 - q_start)) * len(range(0, H, 2))
    assert n_over >= 0.9 * rows, (n_over, rows)
    p.run()
    torch.cuda.synchronize()
    compare(host_f64(p.out), p.oracle(), f"peaked prefill Tq={Tq} H={H}")


def test_prefill_vha_peaked_rows():
    H, rank = 64, 8
    p, n_over = _peaked_prefill(90, 301, H, 200, "f32")
    assert n_over > 1000
    up = (gen(90, synth.CK, (H, rank)) * 0.125).contiguous()
    down = (gen(90, synth.CV, (rank, H)) * 0.125).contiguous()
    hca.hca_compress(p.k_all[:p.Nc * 128], p.v_all[:p.Nc * 128], p.ck, p.cv)
    hca.hca_attn_prefill_vha(p.q, p.g, p.k, p.v, p.ck, p.cv, up, down, p.out,
                             q_start=p.q_start, kv_start=p.kv_start)
    torch.cuda.synchronize()
    want = oracle.vha(p.oracle(), host(up), host(down))
    compare(host_f64(p.out), want, "peaked prefill + VHA")


def test_prefill_peaked_only_late_tile():
    # a single aimed head in a single query: one row of one item takes the
    # exact-maximum path, every other row of every item is ordinary
    p, n_over = _peaked_prefill(91, 640, 16, 0, "f32", heads=[])
    qh, kh = host(p.q), host(p.k_all)
    ck = oracle.compress(kh[:p.Nc * 128])
    t, h = 517, 11
    qh[t, h] = _aim(qh[t, h], kh[t], kh[t - 2])
    assert _gap(qh[t, h], (kh[t], kh[t - 2]), ck[:(t + 1) // 128]) > GAP
    p.q = _to_dev(qh)
    p.run()
    torch.cuda.synchronize()
    compare(host_f64(p.out), p.oracle(), "one peaked row")


def _ring_slot(t):
    return t % 128


@pytest.mark.parametrize("H,out_dtype,B", [(64, "bf16", 8), (16, "f32", 8), (8, "f32", 8),
                                          (64, "f32", 64), (16, "bf16", 256)])
def test_decode_peaked_rows(H, out_dtype, B):
    # positions from 131072 on have at least 64 entry tiles, so every stream of
    # keys (at most 16 splits x 4 waves) starts with an entry tile: the aimed
    # window keys lie more than 2^64 above each stream's first reference
    positions = np.array([5, 130, 300, 140000, 4095, 32768, 150001, 2500], dtype=np.int64)
    positions = np.resize(positions, B)  # larger batches repeat the pattern
    nc_cap = int(max((positions + 1) // 128))
    seed = 92 + H
    q, g = gen(seed, synth.Q, (B, H, D)), gen(seed, synth.G, (B, H, D))
    ck, cv = gen(seed, synth.CK, (B, nc_cap, D)), gen(seed, synth.CV, (B, nc_cap, D))
    wk, wv = gen(seed, synth.WK, (B, 128, D)), gen(seed, synth.WV, (B, 128, D))
    qh, wkh, ckh = host(q), host(wk), host(ck)
    n_over = n_late = 0
    for b, t in enumerate(positions):
        nc = (t + 1) // 128
        if nc == 0:
            continue
        for h in range(0, H, 2):
            ka, kb = wkh[b, _ring_slot(t)], wkh[b, _ring_slot(t - 5)]
            qh[b, h] = _aim(qh[b, h], ka, kb)
            over = _gap(qh[b, h], (ka, kb), ckh[b, :nc]) > GAP
            n_over += over
            n_late += over and nc >= 1024
    assert n_over >= 0.9 * (B * 7 // 8) * max(1, H // 2), n_over
    assert n_late >= 2 * max(1, H // 2), n_late
    q = _to_dev(qh)
    pos = torch.as_tensor(positions, device=dev())
    out = torch.empty((B, H, D), device=dev(),
                      dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16)
    hca.hca_attn_decode(q, g, ck, cv, wk, wv, pos, out)
    torch.cuda.synchronize()
    ref = oracle.decode(qh, host(g), ckh, host(cv), wkh, host(wv), positions)
    compare(host_f64(out), ref, f"peaked decode H={H}")


@pytest.mark.parametrize("M,H", [(3, 64), (2, 16), (3, 8), (2, 24)])
def test_decode_multi_peaked_rows(M, H):
    positions = np.array([3, 129, 700, 32765, 5000], dtype=np.int64)
    B = len(positions)
    nc_cap = int(max((positions + M) // 128))
    seed = 95 + M
    q, g = gen(seed, synth.Q, (B, M, H, D)), gen(seed, synth.G, (B, M, H, D))
    ck, cv = gen(seed, synth.CK, (B, nc_cap, D)), gen(seed, synth.CV, (B, nc_cap, D))
    wk, wv = gen(seed, synth.WK, (B, 128, D)), gen(seed, synth.WV, (B, 128, D))
    nk, nv = gen(seed, synth.NK, (B, M, D)), gen(seed, synth.NV, (B, M, D))
    qh, wkh, ckh, nkh = host(q), host(wk), host(ck), host(nk)
    n_over = n_late = 0
    for b, t in enumerate(positions):
        for j in range(M):
            nc = (t + j + 1) // 128
            if nc == 0:
                continue
            for h in range(1, H, 2):
                # the token's own new row and a committed ring row of its window
                ka, kb = nkh[b, j], wkh[b, _ring_slot(t - 2)]
                qh[b, j, h] = _aim(qh[b, j, h], ka, kb)
                over = _gap(qh[b, j, h], (ka, kb), ckh[b, :nc]) > GAP
                n_over += over
                # 64 entries or more: each of the 4 key streams starts with an entry tile
                n_late += over and nc >= 64
    assert n_over >= 0.9 * 4 * M * (H // 2), n_over
    assert n_late >= M * (H // 2), n_late
    q = _to_dev(qh)
    pos = torch.as_tensor(positions, device=dev())
    out = torch.empty((B, M, H, D), device=dev(), dtype=torch.float32)
    hca.hca_attn_decode_multi(q, g, ck, cv, wk, wv, nk, nv, pos, out)
    torch.cuda.synchronize()
    ref = oracle.decode_multi(qh, host(g), ckh, host(cv), wkh, host(wv), nkh, host(nv),
                              positions)
    compare(host_f64(out), ref, f"peaked decode_multi M={M} H={H}")
