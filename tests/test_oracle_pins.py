"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

The oracle never checks itself here: each test compares it with a different
computation (dense masked brute force, exact rationals, torch SDPA, closed
forms, or a second oracle entry point with different indexing).
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from tests._independent import (dense_masked_attention, exact_block_mean_bf16, sdpa_causal,
                                widen)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _problem(seed, T, H, D, block, *, q_start=0, kv_start=0, Tq=None):
    """Seeded inputs for positions [0, T): queries q_start..q_start+Tq-1."""
    Tq = T - q_start if Tq is None else Tq
    k = synth.normal_bf16(seed, synth.K, (T, D))
    v = synth.normal_bf16(seed, synth.V, (T, D))
    q = synth.normal_bf16(seed, synth.Q, (Tq, H, D))
    g = synth.normal_bf16(seed, synth.G, (Tq, H, D))
    return q, g, k, v


# ---------------------------------------------------------------- compress
def test_compress_matches_exact_rational_mean(oracle_mod):
    # block entry = mean of the block's rows, stored as bf16 (nearest, ties to even)
    for block, T, D in [(4, 18, 6), (128, 256, 3)]:
        x = synth.normal_bf16(11, synth.K, (T, D))
        got = oracle_mod.compress(x, block)
        want = exact_block_mean_bf16(x, block)
        assert got.shape == (T // block, D)
        for b in range(T // block):
            for d in range(D):
                assert Fraction(float(widen(got[b, d]))) == want[b][d], (block, b, d)


def test_compress_closed_forms(oracle_mod):
    D = 16
    c = synth.normal_bf16(5, synth.K, (1, D))
    const = np.repeat(c, 256, axis=0)
    assert np.array_equal(oracle_mod.compress(const, 128), np.repeat(c, 2, axis=0))
    # arithmetic progression a + i*delta over one block: mean = a + 127*delta/2, exact
    i = np.arange(128, dtype=np.float64)[:, None]
    a, delta = 3.0, 0.25
    prog = synth.f32_to_bf16_bits((a + i * delta) * np.ones((1, D)))
    assert np.all(widen(prog) == a + i * delta)  # inputs exactly representable
    assert np.all(widen(oracle_mod.compress(prog, 128)) == a + 127 * delta / 2)
    # order within a block does not matter; a trailing partial block is dropped
    x = synth.normal_bf16(6, synth.V, (300, D))
    perm = np.concatenate([np.random.default_rng(0).permutation(128), 128 + np.arange(172)])
    assert np.array_equal(oracle_mod.compress(x, 128), oracle_mod.compress(x[perm], 128))
    assert oracle_mod.compress(x, 128).shape == (2, D)


def test_round_bf16_ties_to_even(oracle_mod):
    # 1 + 2^-8 is half way between 1 and 1 + 2^-7 -> even (1.0);
    # 1 + 3*2^-8 is half way between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    assert oracle_mod.round_bf16(1 + 2 ** -8) == 0x3F80
    assert oracle_mod.round_bf16(1 + 3 * 2 ** -8) == 0x3F82
    assert oracle_mod.round_bf16(-(1 + 3 * 2 ** -8)) == 0xBF82
    assert oracle_mod.round_bf16(1 + 2 ** -8 + 2 ** -30) == 0x3F81
    assert oracle_mod.round_bf16(2.0 ** -133) == 0x0001          # smallest subnormal
    assert oracle_mod.round_bf16(2.0 ** -134) == 0x0000          # tie -> even (zero)
    assert oracle_mod.round_bf16(3.0 * 2.0 ** -135) == 0x0001
    assert oracle_mod.round_bf16(2.0 ** 128) == 0x7F80           # overflow -> inf
    assert oracle_mod.round_bf16((2 - 2 ** -7) * 2.0 ** 127) == 0x7F7F
    for b in [0x0001, 0x3F80, 0xC2F7, 0x7F7F, 0x8080]:
        assert oracle_mod.round_bf16(oracle_mod.widen_bf16(b)) == b


# ---------------------------------------------------------------- attention
@pytest.mark.parametrize("block,window,D,H,T", [(4, 4, 8, 2, 64), (4, 6, 8, 3, 50),
                                                (8, 4, 5, 1, 41)])
def test_attn_equals_dense_brute_force_small_blocks(oracle_mod, block, window, D, H, T):
    q, g, k, v = _problem(21 + T, T, H, D, block)
    ck, cv = oracle_mod.compress(k, block), oracle_mod.compress(v, block)
    tpos = np.arange(T)
    got = oracle_mod.attn(q, g, tpos, k, v, 0, ck, cv, block=block, window=window, scale=0.37)
    want = dense_masked_attention(q, g, tpos, k, v, 0, ck, cv, block, window, 0.37)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_attn_equals_dense_brute_force_real_constants(oracle_mod):
    # the layer's constants: block = window = 128, D = 512, scale = 1/sqrt(512)
    T, H, D = 600, 2, 512
    q, g, k, v = _problem(3, T, H, D, 128)
    ck, cv = oracle_mod.compress(k), oracle_mod.compress(v)
    rows = sorted({0, 1, 2, 126, 127, 128, 129, 254, 255, 256, 257, 383, 384, 511, 512, 513,
                   598, 599} | set(range(0, T, 37)))
    tpos = np.array(rows)
    got = oracle_mod.attn(q[tpos], g[tpos], tpos, k, v, 0, ck, cv)
    want = dense_masked_attention(q[tpos], g[tpos], tpos, k, v, 0, ck, cv, 128, 128,
                                  1 / np.sqrt(512))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_short_sequence_is_causal_attention(oracle_mod):
    # below 128 tokens no block is complete and the window covers the whole prefix
    T, H, D = 127, 3, 64
    q, g, k, v = _problem(4, T, H, D, 128)
    got = oracle_mod.attn(q, g, np.arange(T), k, v, 0, None, None, scale=0.125)
    want = sdpa_causal(q, g, k, v, 0.125)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # at T = 128 the last query also sees entry 0 (block 0 ends at 127): rows 0..126 stay causal
    T = 128
    q, g, k, v = _problem(5, T, H, D, 128)
    ck, cv = oracle_mod.compress(k), oracle_mod.compress(v)
    got = oracle_mod.attn(q, g, np.arange(T), k, v, 0, ck, cv, scale=0.125)
    np.testing.assert_allclose(got[:127], sdpa_causal(q[:127], g[:127], k[:127], v[:127], 0.125),
                               rtol=0, atol=1e-12)
    nocomp = oracle_mod.attn(q, g, np.arange(T), k, v, 0, None, None, scale=0.125)
    assert np.abs(got[127] - nocomp[127]).max() > 1e-6


def test_row_zero_is_first_value_times_gate(oracle_mod):
    T, H, D = 8, 4, 512
    q, g, k, v = _problem(6, T, H, D, 128)
    got = oracle_mod.attn(q[:1], g[:1], [0], k, v, 0, None, None)
    gate = 1.0 / (1.0 + np.exp(-widen(g[0])))
    np.testing.assert_allclose(got[0], widen(v[0])[None, :] * gate, rtol=1e-15, atol=0)  # numpy exp vs libm exp: an ulp or two


def test_constant_values_give_value_times_gate(oracle_mod):
    T, H, D = 700, 2, 512
    q, g, k, _ = _problem(7, T, H, D, 128)
    c = synth.normal_bf16(7, synth.CV, (1, D))
    v = np.repeat(c, T, axis=0)
    ck, cv = oracle_mod.compress(k), oracle_mod.compress(v)
    assert np.array_equal(cv, np.repeat(c, T // 128, axis=0))
    tpos = np.array([0, 127, 128, 255, 383, 699])
    got = oracle_mod.attn(q[tpos], g[tpos], tpos, k, v, 0, ck, cv)
    want = widen(c)[0][None, None, :] / (1.0 + np.exp(-widen(g[tpos])))
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=0)


def test_gate_limits(oracle_mod):
    T, H, D = 300, 2, 512
    q, g, k, v = _problem(8, T, H, D, 128)
    ck, cv = oracle_mod.compress(k), oracle_mod.compress(v)
    tpos = np.arange(T)
    full = lambda bits: np.full(q.shape, bits, dtype=np.uint16)
    neg_inf = oracle_mod.attn(q, full(0xFF80), tpos, k, v, 0, ck, cv)
    assert np.all(neg_inf == 0.0)                    # sigmoid(-inf) = 0 exactly
    zero = oracle_mod.attn(q, full(0x0000), tpos, k, v, 0, ck, cv)
    pos_inf = oracle_mod.attn(q, full(0x7F80), tpos, k, v, 0, ck, cv)
    assert np.array_equal(2.0 * zero, pos_inf)       # sigmoid(0) = 1/2, sigmoid(+inf) = 1
    ungated = dense_masked_attention(q, full(0x7F80), tpos, k, v, 0, ck, cv, 128, 128,
                                     1 / np.sqrt(D))
    np.testing.assert_allclose(pos_inf, ungated, rtol=0, atol=1e-12)


def test_zero_query_averages_visible_values(oracle_mod):
    # q = 0 makes every score 0, so the output is the plain mean of the visible values
    T, H, D, block, window = 520, 1, 16, 128, 128
    _, _, k, v = _problem(9, T, H, D, block)
    q = np.zeros((T, H, D), np.uint16)
    g = np.full((T, H, D), 0x7F80, np.uint16)
    ck, cv = oracle_mod.compress(k), oracle_mod.compress(v)
    got = oracle_mod.attn(q, g, np.arange(T), k, v, 0, ck, cv)
    vf, cvf = widen(v), widen(cv)
    for t in [0, 1, 126, 127, 128, 129, 254, 255, 256, 300, 383, 384, 511, 512, 519]:
        n_entries = (t + 1) // block                 # blocks whose last token is <= t
        first = max(0, t - window + 1)
        rows = np.concatenate([cvf[:n_entries], vf[first:t + 1]])
        assert rows.shape[0] == n_entries + min(t + 1, window)
        np.testing.assert_allclose(got[t, 0], rows.mean(axis=0), rtol=1e-13, atol=1e-15)


def _golden(name):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        return json.load(f)


def test_worked_example_uniform_weights(oracle_mod):
    # Hand-derived example (tests/golden/worked_uniform_weights.json): q = 0, G = 0.
    gd = _golden("worked_uniform_weights.json")
    T, D = len(gd["v"]), gd["D"]
    v = synth.f32_to_bf16_bits(np.array(gd["v"], dtype=np.float32))
    k = synth.f32_to_bf16_bits(np.array(gd["k"], dtype=np.float32))
    q = np.zeros((T, 1, D), np.uint16)
    g = np.zeros((T, 1, D), np.uint16)
    b = gd["block"]
    ck, cv = oracle_mod.compress(k, b), oracle_mod.compress(v, b)
    got = oracle_mod.attn(q, g, np.arange(T), k, v, 0, ck, cv, block=b, window=gd["window"],
                          scale=gd["scale"])
    want = np.array([[float(Fraction(x)) for x in row] for row in gd["expected"]])
    np.testing.assert_allclose(got[:, 0, :], want, rtol=1e-15, atol=1e-15)


def test_worked_example_softmax_weights(oracle_mod):
    # Hand-derived example (tests/golden/worked_softmax_weights.json): q = 1, G = +inf;
    # expected value of row t = sum_j e^{s_j} v_j / sum_j e^{s_j} over its (s_j, v_j).
    gd = _golden("worked_softmax_weights.json")
    want = [sum(np.exp(s) * val for s, val in terms) / sum(np.exp(s) for s, _ in terms)
            for terms in gd["expected_terms"]]
    T, b = len(gd["k"]), gd["block"]
    k = synth.f32_to_bf16_bits(np.array(gd["k"], np.float32))
    v = synth.f32_to_bf16_bits(np.array(gd["v"], np.float32))
    q = synth.f32_to_bf16_bits(np.ones((T, 1, 1), np.float32))
    g = np.full((T, 1, 1), 0x7F80, np.uint16)
    ck, cv = oracle_mod.compress(k, b), oracle_mod.compress(v, b)
    got = oracle_mod.attn(q, g, np.arange(T), k, v, 0, ck, cv, block=b, window=gd["window"],
                          scale=gd["scale"])
    np.testing.assert_allclose(got[:, 0, 0], want, rtol=1e-14)


def test_oracle_regression_fixture():
    # Records the oracle (not an independent pin): tests/golden/make_oracle_fixture.py
    import importlib.util
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "make_oracle_fixture.py")
    spec = importlib.util.spec_from_file_location("make_oracle_fixture", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    gd = _golden("oracle_regression_small.json")
    want = np.array([float.fromhex(x) for x in gd["out"]])
    np.testing.assert_array_equal(mod.compute().ravel(), want)


# ---------------------------------------------------------------- cross-entry identities
def test_chunk_equals_monolithic(oracle_mod):
    T, H, D = 700, 2, 64
    q, g, k, v = _problem(10, T, H, D, 128)
    ck, cv = oracle_mod.compress(k), oracle_mod.compress(v)
    full = oracle_mod.attn(q, g, np.arange(T), k, v, 0, ck, cv)
    a = 300                                  # chunk of queries 300..699 with K/V from 173
    kv0 = a - 127
    part = oracle_mod.attn(q[a:], g[a:], np.arange(a, T), k[kv0:], v[kv0:], kv0, ck, cv)
    assert np.array_equal(part, full[a:])


def test_decode_equals_prefill_row(oracle_mod):
    T, H, D, W = 900, 2, 64, 128
    q, g, k, v = _problem(12, T, H, D, 128)
    ck, cv = oracle_mod.compress(k), oracle_mod.compress(v)
    positions = np.array([0, 5, 126, 127, 128, 255, 256, 640, 899])
    B = len(positions)
    nc_cap = 8
    ckb = np.zeros((B, nc_cap, D), np.uint16)
    cvb = np.zeros((B, nc_cap, D), np.uint16)
    wk = np.zeros((B, W, D), np.uint16)
    wv = np.zeros((B, W, D), np.uint16)
    for b, t in enumerate(positions):
        n = (t + 1) // 128
        ckb[b, :n], cvb[b, :n] = ck[:n], cv[:n]
        for p in range(max(0, t - W + 1), t + 1):
            wk[b, p % W], wv[b, p % W] = k[p], v[p]
    dec = oracle_mod.decode(q[positions], g[positions], ckb, cvb, wk, wv, positions)
    pre = oracle_mod.attn(q, g, np.arange(T), k, v, 0, ck, cv)
    assert np.array_equal(dec, pre[positions])


def test_range_errors(oracle_mod):
    T, H, D = 300, 1, 8
    q, g, k, v = _problem(13, T, H, D, 128)
    with pytest.raises(oracle_mod.OracleError):      # raw row 73 needed, K starts at 100
        oracle_mod.attn(q[200:201], g[200:201], [200], k[100:], v[100:], 100, None, None)
    with pytest.raises(oracle_mod.OracleError):      # position 300 beyond the raw rows
        oracle_mod.attn(q[:1], g[:1], [300], k, v, 0, None, None)
