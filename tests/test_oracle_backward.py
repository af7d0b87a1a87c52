"""Pins of the oracle's backward pass (``oracle.attn_backward``), independent of
it: central finite differences of an fp64 forward written separately
(tests/_independent.py), torch autograd on an fp64 dense masked attention,
closed forms of the gate, and planted mistakes that the battery must catch.
CPU only."""
import ctypes
import subprocess

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._independent import dense_attention_f64, widen

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _dyadic(seed, shape, lo=-16, hi=16):
    """bf16 bits of multiples of 1/8 in [lo/8, hi/8]: block means of four such rows
    are exact in bf16, so the oracle's rounded entries equal the exact means."""
    rng = np.random.default_rng(seed)
    x = rng.integers(lo, hi + 1, size=shape).astype(np.float32) / 8
    return synth.f32_to_bf16_bits(x)


def _inputs(seed, T, H, D):
    q = synth.normal_bf16(seed, synth.Q, (T, H, D))
    g = synth.normal_bf16(seed, synth.G, (T, H, D))
    do = synth.normal_bf16(seed, 12, (T, H, D))
    k, v = _dyadic(seed, (T, D)), _dyadic(seed + 1, (T, D))
    return q, g, do, k, v


def _fd_check(q, g, do, k, v, block, window, scale, n_coords=24, seed=0):
    """Central differences of L = sum(dO * out) at random coordinates of q, g, k,
    v against the oracle's gradients.  Returns the worst relative error."""
    dq, dk, dv, dg = oracle.attn_backward(q, g, do, k, v, block=block, window=window,
                                          scale=scale)
    base = dict(q=widen(q), g=widen(g), k=widen(k), v=widen(v))
    dof = widen(do)
    grads = dict(q=dq, g=dg, k=dk, v=dv)
    rng = np.random.default_rng(seed)
    worst = 0.0
    h = 1e-6

    def loss(x):
        out = dense_attention_f64(x["q"], x["g"], x["k"], x["v"], block, window, scale)
        return float((dof * out).sum())

    for name, arr in base.items():
        for _ in range(n_coords):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            xp = {kk: vv.copy() for kk, vv in base.items()}
            xm = {kk: vv.copy() for kk, vv in base.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            fd = (loss(xp) - loss(xm)) / (2 * h)
            an = grads[name][idx]
            worst = max(worst, abs(fd - an) / max(1e-3, abs(fd)))
    return worst


def test_finite_differences_small_blocks():
    # block = window = 4, D = 8: entries, window edges and ragged tails all occur
    q, g, do, k, v = _inputs(1, 23, 2, 8)
    assert _fd_check(q, g, do, k, v, 4, 4, 0.35) < 1e-6


def test_finite_differences_window_longer_than_block():
    q, g, do, k, v = _inputs(2, 30, 3, 8)
    assert _fd_check(q, g, do, k, v, 4, 7, 0.3, seed=1) < 1e-6


def _torch_reference(q, g, do, k, v, block, window, scale):
    """fp64 autograd through a dense masked attention whose entries are the block
    means of k and v (in the graph, so their gradients reach every row)."""
    qf, gf, kf, vf = (torch.tensor(widen(x), requires_grad=True) for x in (q, g, k, v))
    T, H, D = qf.shape
    nc = T // block
    ck = kf[:nc * block].reshape(nc, block, D).mean(1)
    cv = vf[:nc * block].reshape(nc, block, D).mean(1)
    kaug, vaug = torch.cat([kf, ck]), torch.cat([vf, cv])
    pos = torch.arange(T)
    t = pos[:, None]
    vis = torch.cat([(pos[None] <= t) & (pos[None] > t - window),
                     (torch.arange(nc) * block + block - 1)[None] <= t], dim=1)
    s = scale * torch.einsum("thd,jd->thj", qf, kaug)
    s = s.masked_fill(~vis[:, None, :], float("-inf"))
    out = torch.einsum("thj,jd->thd", torch.softmax(s, dim=2), vaug) * torch.sigmoid(gf)
    out.backward(torch.tensor(widen(do)))
    return qf.grad.numpy(), kf.grad.numpy(), vf.grad.numpy(), gf.grad.numpy()


def test_torch_autograd_real_constants():
    # block = window = 128, T = 300: two entries; K and V constant within each
    # 128-row block, so the oracle's bf16 entries are the exact means
    T, H, D = 300, 2, 32
    q = synth.normal_bf16(3, synth.Q, (T, H, D))
    g = synth.normal_bf16(3, synth.G, (T, H, D))
    do = synth.normal_bf16(3, 12, (T, H, D))
    kb = synth.normal_bf16(3, synth.K, (3, D))
    vb = synth.normal_bf16(3, synth.V, (3, D))
    k = np.repeat(kb, 128, axis=0)[:T].copy()
    v = np.repeat(vb, 128, axis=0)[:T].copy()
    got = oracle.attn_backward(q, g, do, k, v, scale=D ** -0.5)
    want = _torch_reference(q, g, do, k, v, 128, 128, D ** -0.5)
    for a, b, name in zip(got, want, ["dq", "dk", "dv", "dg"]):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-11, err_msg=name)


def test_torch_autograd_causal_only():
    # T <= 127 with window 128: plain causal attention, no entries
    T, H, D = 100, 3, 16
    q, g, do = (synth.normal_bf16(4, i, (T, H, D)) for i in (synth.Q, synth.G, 12))
    k, v = synth.normal_bf16(4, synth.K, (T, D)), synth.normal_bf16(4, synth.V, (T, D))
    got = oracle.attn_backward(q, g, do, k, v, scale=0.25)
    want = _torch_reference(q, g, do, k, v, 128, 128, 0.25)
    for a, b, name in zip(got, want, ["dq", "dk", "dv", "dg"]):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-11, err_msg=name)


def test_gate_closed_forms():
    T, H, D = 40, 2, 8
    q, g, do, k, v = _inputs(5, T, H, D)
    # sigmoid(+inf) = 1: the gate's own gradient sig (1 - sig) is exactly 0
    dq, dk, dv, dg = oracle.attn_backward(q, np.full(q.shape, 0x7F80, np.uint16), do, k, v,
                                          block=4, window=4)
    assert np.all(dg == 0)
    # sigmoid(-inf) = 0: nothing reaches the attention and the gate's gradient is 0
    grads = oracle.attn_backward(q, np.full(q.shape, 0xFF80, np.uint16), do, k, v, block=4,
                                 window=4)
    assert all(np.all(x == 0) for x in grads)
    # no upstream gradient: every gradient is 0
    grads = oracle.attn_backward(q, g, np.zeros_like(do), k, v, block=4, window=4)
    assert all(np.all(x == 0) for x in grads)


def test_values_gradient_sums_to_upstream():
    # each row's weights sum to 1, so the value gradients (raw rows plus entries,
    # before pooling) add up to the sum over rows of dO * sigmoid(g)
    T, H, D = 37, 2, 8
    q, g, do, k, v = _inputs(6, T, H, D)
    _, _, dv, _ = oracle.attn_backward(q, g, do, k, v, block=4, window=4)
    want = (widen(do) / (1 + np.exp(-widen(g)))).sum(axis=(0, 1))
    np.testing.assert_allclose(dv.sum(axis=0), want, rtol=1e-12, atol=1e-12)


MUTANTS = {
    "no_softmax_centering": ("const double ds = p[j] * (dp[j] - dsum);",
                             "const double ds = p[j] * dp[j];"),
    "ds_without_weight": ("const double ds = p[j] * (dp[j] - dsum);",
                          "const double ds = (dp[j] - dsum);"),
    "dk_without_scale": ("akj[d] += scale * ds * widen_bf16(q[off + d]);",
                         "akj[d] += ds * widen_bf16(q[off + d]);"),
    "dv_from_scores": ("avj[d] += p[j] * da[d];", "avj[d] += ds * da[d];"),
    "gate_grad_sign": ("dg[off + d] = go * a[d] * sig * (1.0 - sig);",
                       "dg[off + d] = go * a[d] * sig * (1.0 + sig);"),
    "ungated_upstream": ("da[d] = go * sig;", "da[d] = go;"),
    "entries_not_seen": ("kid[nk] = T + b;", "kid[nk] = b;"),
}


@pytest.fixture()
def mutant(tmp_path, request, monkeypatch):
    name = request.param
    src = open(oracle.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path_c = tmp_path / f"{name}.c"
    path_c.write_text(src.replace(old, new))
    path_so = tmp_path / f"{name}.so"
    subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared",
                           "-ffp-contract=off", str(path_c), "-o", str(path_so), "-lm"])
    monkeypatch.setattr(oracle, "_lib", oracle.bind(ctypes.CDLL(str(path_so))))
    return name


@pytest.mark.parametrize("mutant", sorted(MUTANTS), indirect=True)
def test_backward_mutant_is_caught(mutant):
    q, g, do, k, v = _inputs(1, 23, 2, 8)
    assert _fd_check(q, g, do, k, v, 4, 4, 0.35, n_coords=12) > 1e-4, mutant


def test_rows_equal_the_full_routine():
    # the row-sampled entry point runs the same per-row code: bit for bit the rows
    # of the whole-sequence result, for positions around block and window edges
    T, H, D = 700, 3, 64
    q, g, do, k, v = _inputs(21, T, H, D)
    dq, _, _, dg = oracle.attn_backward(q, g, do, k, v, scale=0.125)
    pos = np.array([0, 1, 126, 127, 128, 255, 256, 383, 511, 600, 699], dtype=np.int64)
    dq_r, dg_r = oracle.attn_backward_rows(q[pos], g[pos], do[pos], pos, k, v, scale=0.125)
    np.testing.assert_array_equal(dq_r, dq[pos])
    np.testing.assert_array_equal(dg_r, dg[pos])


def test_key_gradient_sums():
    # sum_j ds_j = 0 for every row, so the key gradients sum to zero; the weights
    # sum to one, so the value gradients sum to sum over rows of dO * sigmoid(g)
    # (both through the entries too: an entry's gradient reaches its block's rows
    # divided by the block size, which keeps the sums)
    T, H, D = 600, 2, 32
    q, g, do, k, v = _inputs(22, T, H, D)
    _, dk, dv, _ = oracle.attn_backward(q, g, do, k, v, scale=0.3)
    gf, dof = widen(g), widen(do)
    want_v = (dof / (1.0 + np.exp(-gf))).sum(axis=(0, 1))
    np.testing.assert_allclose(dv.sum(axis=0), want_v, rtol=1e-10, atol=1e-10)
    assert np.abs(dk.sum(axis=0)).max() <= 1e-10 * np.abs(dk).sum()


# ---- the forward's row log-sum-exp and the backward from saved state


def _dense_lse(q, tpos, k, kv_start, ck, block, window, scale):
    """Brute force: scores against one dense key matrix with a boolean visibility
    mask, then numpy's maximum-shifted log of the summed exponentials."""
    kaug = np.concatenate([widen(k), widen(ck)], axis=0)
    raw_pos = kv_start + np.arange(k.shape[0])
    block_last = np.arange(ck.shape[0]) * block + (block - 1)
    t = np.asarray(tpos, dtype=np.int64)[:, None]
    vis = np.concatenate([(raw_pos[None] <= t) & (raw_pos[None] > t - window),
                          block_last[None] <= t], axis=1)
    s = scale * np.einsum("nhd,jd->nhj", widen(q), kaug)
    s = np.where(vis[:, None, :], s, -np.inf)
    top = s.max(axis=2)
    return top + np.log(np.exp(s - top[..., None]).sum(axis=2))


def test_lse_against_brute_force():
    T, H, D = 45, 3, 8
    q, _, _, k, _ = _inputs(31, T, H, D)
    ck = oracle.compress(k, 4)
    pos = np.arange(T)
    got = oracle.attn_lse(q, pos, k, 0, ck, block=4, window=5, scale=0.4)
    np.testing.assert_allclose(got, _dense_lse(q, pos, k, 0, ck, 4, 5, 0.4), rtol=1e-13,
                               atol=1e-13)
    # a chunk of later queries whose raw rows start past position 0
    pos2 = np.arange(30, 45)
    got2 = oracle.attn_lse(q[30:], pos2, k[26:], 26, ck, block=4, window=5, scale=0.4)
    np.testing.assert_allclose(got2, got[30:], rtol=1e-13, atol=1e-13)


def test_lse_of_zero_queries_counts_the_visible_keys():
    # q = 0: every score is 0, so lse = ln(number of keys the row sees), which
    # pins the two visibility rules at block and window edges
    T, H, D, block, window = 50, 2, 8, 4, 6
    q = np.zeros((T, H, D), np.uint16)
    k = _dyadic(32, (T, D))
    ck = oracle.compress(k, block)
    lse = oracle.attn_lse(q, np.arange(T), k, 0, ck, block=block, window=window, scale=1.0)
    for t in range(T):
        n = min(t + 1, window) + (t + 1) // block
        np.testing.assert_allclose(lse[t], np.log(n), rtol=0, atol=1e-14)


def _exact_state(q, g, k, v, block, window, scale):
    """The forward's exact gated output and row log-sum-exp (oracle, fp64)."""
    T = q.shape[0]
    ck, cv = oracle.compress(k, block), oracle.compress(v, block)
    pos = np.arange(T)
    out = oracle.attn(q, g, pos, k, v, 0, ck, cv, block=block, window=window, scale=scale)
    lse = oracle.attn_lse(q, pos, k, 0, ck, block=block, window=window, scale=scale)
    return out, lse


def test_saved_state_backward_is_the_exact_gradient():
    # with the exact output and log-sum-exp, D = <dO, o> = <dA, a> and the
    # weights exp(x - lse) are the softmax: the exact gradients, which finite
    # differences and torch autograd pin above
    T, H, D, block, window, scale = 41, 2, 8, 4, 5, 0.35
    q, g, do, k, v = _inputs(33, T, H, D)
    out, lse = _exact_state(q, g, k, v, block, window, scale)
    got = oracle.attn_backward_saved(q, g, do, out, lse, k, v, block=block, window=window,
                                     scale=scale)
    want = oracle.attn_backward(q, g, do, k, v, block=block, window=window, scale=scale)
    for a, b, name in zip(got, want, ["dq", "dk", "dv", "dg"]):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12, err_msg=name)


def test_saved_state_closed_forms():
    T, H, D, block, window, scale = 30, 2, 8, 4, 4, 0.3
    q, g, do, k, v = _inputs(34, T, H, D)
    out, lse = _exact_state(q, g, k, v, block, window, scale)
    base = oracle.attn_backward_saved(q, g, do, out, lse, k, v, block=block, window=window,
                                      scale=scale)
    # lse raised by delta scales every weight, so dq, dk, dv, by exp(-delta);
    # dg does not involve the weights
    shifted = oracle.attn_backward_saved(q, g, do, out, lse + 0.5, k, v, block=block,
                                         window=window, scale=scale)
    for a, b in zip(shifted[:3], base[:3]):
        np.testing.assert_allclose(a, b * np.exp(-0.5), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(shifted[3], base[3])
    # a gate of logit 40 has sigmoid exactly 1 in fp64: dA = dO is already a
    # bfloat16 value, so rounding it changes nothing, and dg = dO o (1 - 1) = 0
    g40 = np.full(q.shape, 0x4220, np.uint16)
    plain = oracle.attn_backward_saved(q, g40, do, out, lse, k, v, block=block, window=window,
                                       scale=scale)
    rounded = oracle.attn_backward_saved(q, g40, do, out, lse, k, v, round_da=True, block=block,
                                         window=window, scale=scale)
    for a, b in zip(plain, rounded):
        np.testing.assert_array_equal(a, b)
    assert np.all(plain[3] == 0)
    # rounding dA is the same as passing the rounded product as dout with that
    # gate; dv = sum of weights times dA is the gradient that involves dA alone
    gf, dof = widen(g), widen(do)
    da_bits = synth.f64_to_bf16_bits(dof / (1.0 + np.exp(-gf)))
    r1 = oracle.attn_backward_saved(q, g, do, out, lse, k, v, round_da=True, block=block,
                                    window=window, scale=scale)
    r2 = oracle.attn_backward_saved(q, g40, da_bits, out, lse, k, v, block=block, window=window,
                                    scale=scale)
    np.testing.assert_allclose(r1[2], r2[2], rtol=1e-12, atol=1e-14)


SAVED_MUTANTS = {
    "saved_d_from_da": ("dsum_o += up * o[off + d];", "dsum_o += up * s_g * o[off + d];"),
    "saved_weights_ignore_lse": ("const double pj = exp(scale * qk - lse);",
                                 "const double pj = exp(scale * qk);"),
    "saved_gate_grad_with_sigmoid": ("dg[off + d] = up * o[off + d] * (1.0 - s_g);",
                                     "dg[off + d] = up * o[off + d] * s_g * (1.0 - s_g);"),
    "saved_dk_from_v": ("gk[(size_t)acc_row * D + d] += scale * dsj * widen_bf16(q[off + d]);",
                        "gk[(size_t)acc_row * D + d] += scale * dsj * widen_bf16(vr[d]);"),
    "saved_window_short": ("const int64_t w0 = t - window + 1 < 0 ? 0 : t - window + 1;",
                           "const int64_t w0 = t - window + 2 < 0 ? 0 : t - window + 2;"),
}


@pytest.fixture()
def saved_mutant(tmp_path, request, monkeypatch):
    name = request.param
    src = open(oracle.SRC).read()
    old, new = SAVED_MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path_c = tmp_path / f"{name}.c"
    path_c.write_text(src.replace(old, new))
    path_so = tmp_path / f"{name}.so"
    subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared",
                           "-ffp-contract=off", str(path_c), "-o", str(path_so), "-lm"])
    monkeypatch.setattr(oracle, "_lib", oracle.bind(ctypes.CDLL(str(path_so))))
    return name


@pytest.mark.parametrize("saved_mutant", sorted(SAVED_MUTANTS), indirect=True)
def test_saved_state_mutant_is_caught(saved_mutant):
    T, H, D, block, window, scale = 23, 2, 8, 4, 4, 0.35
    q, g, do, k, v = _inputs(35, T, H, D)
    out, lse = _exact_state(q, g, k, v, block, window, scale)
    got = oracle.attn_backward_saved(q, g, do, out, lse, k, v, block=block, window=window,
                                     scale=scale)
    want = oracle.attn_backward(q, g, do, k, v, block=block, window=window, scale=scale)
    worst = max(float(np.abs(a - b).max() / np.abs(b).max()) for a, b in zip(got, want))
    assert worst > 1e-6, saved_mutant
