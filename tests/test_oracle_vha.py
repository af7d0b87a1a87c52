"""Pins of the oracle's VHA head mix: y = (I + up @ down) x over the heads, for
every position and dim.  Checked against closed forms (zero rank term,
single-entry factors), a pure-Python triple loop on a tiny case, and the
composition with attention; planted mistakes in a copy must each fail."""
import inspect
import textwrap

import numpy as np
import pytest

import synth
from tests._independent import widen


def _x(seed, T, H, D):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, H, D))


def _bits(vals):
    return synth.f64_to_bf16_bits(np.asarray(vals, dtype=np.float64))


def test_zero_factor_is_identity(oracle_mod):
    x = _x(1, 3, 8, 16)
    up = _bits(np.zeros((8, 4)))
    down = synth.normal_bf16(1, synth.G, (4, 8))
    assert np.array_equal(oracle_mod.vha(x, up, down), x)


def test_single_entries_add_one_head_to_another(oracle_mod):
    # up = e_i (rank 1), down = e_j: head i gains head j, every other head is unchanged
    H, i, j = 8, 5, 2
    x = _x(2, 4, H, 16)
    up = np.zeros((H, 1)); up[i, 0] = 1.0
    down = np.zeros((1, H)); down[0, j] = 1.0
    y = oracle_mod.vha(x, _bits(up), _bits(down))
    want = x.copy()
    want[:, i] += x[:, j]
    assert np.array_equal(y, want)


def test_scaled_entries(oracle_mod):
    # up[i, 0] = 0.5, down[0, j] = -2, down[0, i] = 0.25: y_i = x_i + 0.5 (0.25 x_i - 2 x_j)
    H, i, j = 4, 3, 0
    x = _x(3, 2, H, 8)
    up = np.zeros((H, 2)); up[i, 0] = 0.5
    down = np.zeros((2, H)); down[0, j] = -2.0; down[0, i] = 0.25; down[1, :] = 7.0
    y = oracle_mod.vha(x, _bits(up), _bits(down))
    want = x.copy()
    want[:, i] = x[:, i] + 0.5 * (0.25 * x[:, i] - 2.0 * x[:, j])
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-15)


def test_triple_loop(oracle_mod):
    T, H, D, r = 2, 5, 3, 3
    x = _x(4, T, H, D)
    up = synth.normal_bf16(4, synth.Q, (H, r))
    down = synth.normal_bf16(4, synth.K, (r, H))
    U, W = widen(up), widen(down)
    want = np.zeros_like(x)
    for t in range(T):
        for h in range(H):
            for d in range(D):
                acc = x[t, h, d]
                for k in range(r):
                    zk = 0.0
                    for h2 in range(H):
                        zk += W[k, h2] * x[t, h2, d]
                    acc += U[h, k] * zk
                want[t, h, d] = acc
    np.testing.assert_allclose(oracle_mod.vha(x, up, down), want, rtol=1e-13, atol=1e-13)


def test_composition_with_attention(oracle_mod):
    T, H, D = 300, 4, 64
    k = synth.normal_bf16(5, synth.K, (T, D))
    v = synth.normal_bf16(5, synth.V, (T, D))
    q = synth.normal_bf16(5, synth.Q, (T, H, D))
    g = synth.normal_bf16(5, synth.G, (T, H, D))
    ck, cv = oracle_mod.compress(k), oracle_mod.compress(v)
    up = synth.normal_bf16(5, synth.CK, (H, 2))
    down = synth.normal_bf16(5, synth.CV, (2, H))
    tp = np.arange(T)
    a = oracle_mod.attn(q, g, tp, k, v, 0, ck, cv)
    y = oracle_mod.attn_vha(q, g, tp, k, v, 0, ck, cv, up, down)
    np.testing.assert_allclose(y, a + np.einsum("hk,kj,tjd->thd", widen(up), widen(down), a),
                               rtol=1e-12, atol=1e-12)


MUTANTS = {
    "no_identity": ("return x + np.einsum", "return 0 * x + np.einsum"),
    "factors_swapped": ('z = np.einsum("kh,thd->tkd", W, x)', 'z = np.einsum("hk,thd->tkd", U, x)'),
    "up_transposed": ('np.einsum("hk,tkd->thd", U, z)', 'np.einsum("kh,tkd->thd", W, z)'),
    "mix_over_dims": ('z = np.einsum("kh,thd->tkd", W, x)',
                      'z = np.einsum("kh,thd->tkd", W, x[:, :, ::-1])'),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(oracle_mod, name, monkeypatch):
    src = textwrap.dedent(inspect.getsource(oracle_mod.vha))
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    ns = dict(vars(oracle_mod))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(oracle_mod, "vha", ns["vha"])
    failed = 0
    for test in (test_zero_factor_is_identity, test_single_entries_add_one_head_to_another,
                 test_scaled_entries, test_triple_loop):
        try:
            test(oracle_mod)
        except (AssertionError, ValueError):
            failed += 1
    assert failed > 0, name
