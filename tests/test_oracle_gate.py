"""Pins of the oracle's low-rank gate (``oracle.gate_logits``,
``oracle.attn_lowrank_gate``): a pure-Python triple loop, one-hot latents that
pick out weight columns, exact agreement with the stored-logit path when the
logits are exact in bfloat16, and the zero-weight closed form.  CPU only."""
import numpy as np

import oracle
import synth
from tests._independent import widen


def _bits(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_triple_loop():
    T, R, N = 3, 5, 6
    lat = synth.normal_bf16(1, 20, (T, R))
    w = synth.normal_bf16(1, 21, (N, R))
    got = oracle.gate_logits(lat, w)
    lf, wf = widen(lat), widen(w)
    for t in range(T):
        for n in range(N):
            acc = 0.0
            for r in range(R):
                acc += float(lf[t, r]) * float(wf[n, r])
            assert abs(got[t, n] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_one_hot_latent_selects_weight_column():
    R, N = 16, 24
    w = synth.normal_bf16(2, 21, (N, R))
    lat = np.zeros((R, R), np.uint16)
    for r in range(R):
        lat[r, r] = 0x3F80  # 1.0
    got = oracle.gate_logits(lat, w)
    np.testing.assert_array_equal(got, widen(w).T)  # row r = column r of W_g


def test_not_transposed():
    # a square, non-symmetric weight: latent @ W^T differs from latent @ W
    R = 8
    w = synth.normal_bf16(3, 21, (R, R))
    lat = synth.normal_bf16(3, 20, (4, R))
    got = oracle.gate_logits(lat, w)
    assert not np.allclose(got, widen(lat) @ widen(w))
    np.testing.assert_allclose(got, widen(lat) @ widen(w).T, rtol=1e-15)


def _attn_inputs(T=300, H=2, D=16, R=8, seed=4):
    q = synth.normal_bf16(seed, synth.Q, (T, H, D))
    k = synth.normal_bf16(seed, synth.K, (T, D))
    v = synth.normal_bf16(seed, synth.V, (T, D))
    ck, cv = oracle.compress(k), oracle.compress(v)
    rng = np.random.default_rng(seed)
    lat = _bits(rng.integers(-2, 3, size=(T, R)))                 # small integers
    w = _bits(rng.integers(-4, 5, size=(H * D, R)) / 8)           # multiples of 1/8
    return q, k, v, ck, cv, lat, w


def test_equals_stored_logits_when_exact_in_bf16():
    q, k, v, ck, cv, lat, w = _attn_inputs()
    T, H, D = q.shape
    G = oracle.gate_logits(lat, w)
    assert np.all(np.abs(G) <= 8) and np.all(G * 8 == np.round(G * 8))  # exact in bf16
    g_bits = _bits(G.reshape(T, H, D))
    want = oracle.attn(q, g_bits, np.arange(T), k, v, 0, ck, cv)
    got = oracle.attn_lowrank_gate(q, lat, w, np.arange(T), k, v, 0, ck, cv)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)


def test_zero_weights_halve_the_attention():
    q, k, v, ck, cv, lat, w = _attn_inputs(seed=5)
    T = q.shape[0]
    got = oracle.attn_lowrank_gate(q, lat, np.zeros_like(w), np.arange(T), k, v, 0, ck, cv)
    ungated = oracle.attn(q, np.full(q.shape, 0x7F80, np.uint16), np.arange(T), k, v, 0, ck, cv)
    np.testing.assert_array_equal(got, ungated / 2)
