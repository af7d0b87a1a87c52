"""Pins of the oracle's multi-token decode (several new tokens per sequence, as in
the verification of a drafter's tokens).

It is composed from the prefill oracle; these tests check it against two other
computations: the single-token decode entry point, one token at a time with the
ring advanced between tokens (different indexing: every row comes from a ring
slot), and the dense masked brute force over the whole sequence.
"""
import numpy as np
import pytest

import synth
from tests._independent import dense_masked_attention

W = 128


def _sequence(seed, T, H, D):
    k = synth.normal_bf16(seed, synth.K, (T, D))
    v = synth.normal_bf16(seed, synth.V, (T, D))
    q = synth.normal_bf16(seed, synth.Q, (T, H, D))
    g = synth.normal_bf16(seed, synth.G, (T, H, D))
    return q, g, k, v


def _state(oracle_mod, k, v, positions, M, nc_cap):
    """Per-sequence caches for new tokens at positions t .. t+M-1: entries of every
    block completed by t+M-1, the ring of committed rows (positions < t), and the
    new rows; the unused ring slots hold rows of no visible position."""
    B, D = len(positions), k.shape[1]
    ck, cv = oracle_mod.compress(k), oracle_mod.compress(v)
    ckb = np.zeros((B, nc_cap, D), np.uint16)
    cvb = np.zeros((B, nc_cap, D), np.uint16)
    wk = np.tile(k[-1:], (B, W, 1))
    wv = np.tile(v[-1:], (B, W, 1))
    nk = np.zeros((B, M, D), np.uint16)
    nv = np.zeros((B, M, D), np.uint16)
    for b, t in enumerate(positions):
        n = (t + M) // 128
        ckb[b, :n], cvb[b, :n] = ck[:n], cv[:n]
        for p in range(max(0, t - W), t):
            wk[b, p % W], wv[b, p % W] = k[p], v[p]
        nk[b], nv[b] = k[t:t + M], v[t:t + M]
    return ckb, cvb, wk, wv, nk, nv


POS = np.array([0, 1, 5, 125, 126, 127, 128, 254, 255, 256, 383, 640, 893])


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_equals_single_token_decode_with_ring_advanced(oracle_mod, M):
    T, H, D = 900, 2, 64
    q, g, k, v = _sequence(40 + M, T, H, D)
    B, nc_cap = len(POS), 8
    ckb, cvb, wk, wv, nk, nv = _state(oracle_mod, k, v, POS, M, nc_cap)
    qm = np.stack([q[t:t + M] for t in POS])
    gm = np.stack([g[t:t + M] for t in POS])
    got = oracle_mod.decode_multi(qm, gm, ckb, cvb, wk, wv, nk, nv, POS)
    rk, rv = wk.copy(), wv.copy()
    for j in range(M):
        for b, t in enumerate(POS):        # write the row of position t+j into its slot
            rk[b, (t + j) % W], rv[b, (t + j) % W] = nk[b, j], nv[b, j]
        one = oracle_mod.decode(qm[:, j], gm[:, j], ckb, cvb, rk, rv, POS + j)
        assert np.array_equal(got[:, j], one), j


def test_equals_dense_brute_force(oracle_mod):
    T, H, D, M = 700, 2, 64, 3
    q, g, k, v = _sequence(47, T, H, D)
    ck, cv = oracle_mod.compress(k), oracle_mod.compress(v)
    positions = np.array([0, 126, 127, 300, 381, 697])
    ckb, cvb, wk, wv, nk, nv = _state(oracle_mod, k, v, positions, M, 6)
    qm = np.stack([q[t:t + M] for t in positions])
    gm = np.stack([g[t:t + M] for t in positions])
    got = oracle_mod.decode_multi(qm, gm, ckb, cvb, wk, wv, nk, nv, positions)
    for b, t in enumerate(positions):
        tp = t + np.arange(M)
        want = dense_masked_attention(q[tp], g[tp], tp, k, v, 0, ck, cv, 128, 128,
                                      1 / np.sqrt(D))
        np.testing.assert_allclose(got[b], want, rtol=0, atol=1e-12)


def test_later_tokens_do_not_change_earlier_ones(oracle_mod):
    # causality among the new tokens: the first M' outputs of an M-token call are
    # the outputs of the M'-token call on the same prefix
    T, H, D = 400, 2, 64
    q, g, k, v = _sequence(48, T, H, D)
    positions = np.array([3, 126, 250])
    outs = {}
    for M in (1, 4):
        ckb, cvb, wk, wv, nk, nv = _state(oracle_mod, k, v, positions, M, 4)
        qm = np.stack([q[t:t + M] for t in positions])
        gm = np.stack([g[t:t + M] for t in positions])
        outs[M] = oracle_mod.decode_multi(qm, gm, ckb, cvb, wk, wv, nk, nv, positions)
    assert np.array_equal(outs[4][:, :1], outs[1])


def test_range_error(oracle_mod):
    D = 8
    z = np.zeros
    with pytest.raises(oracle_mod.OracleError):   # tokens 126..128 need entry 0, nc_cap = 0
        oracle_mod.decode_multi(z((1, 3, 1, D), np.uint16), z((1, 3, 1, D), np.uint16),
                                z((1, 0, D), np.uint16), z((1, 0, D), np.uint16),
                                z((1, W, D), np.uint16), z((1, W, D), np.uint16),
                                z((1, 3, D), np.uint16), z((1, 3, D), np.uint16), [126])


# Planted mistakes in a copy of the composition: each must fail the pins above.
MUTANTS = {
    "ring_slot_off_by_one": ("slots = [p % window", "slots = [(p + 1) % window"),
    "entries_of_first_token_only": ("nc = (t + M) // block", "nc = (t + 1) // block"),
    "new_rows_reversed": ("k = np.concatenate([wk[b, slots], nk[b]])",
                          "k = np.concatenate([wk[b, slots], nk[b][::-1]])"),
    "positions_shifted": ("t + np.arange(M), k, v, lo", "t + np.arange(M) - 1, k, v, lo - 1"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(oracle_mod, name, monkeypatch):
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(oracle_mod.decode_multi))
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    ns = dict(vars(oracle_mod))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(oracle_mod, "decode_multi", ns["decode_multi"])
    failed = 0
    for test in (lambda: test_equals_single_token_decode_with_ring_advanced(oracle_mod, 3),
                 lambda: test_equals_dense_brute_force(oracle_mod)):
        try:
            test()
        except (AssertionError, oracle_mod.OracleError, ValueError, IndexError):
            failed += 1
    assert failed > 0, name
