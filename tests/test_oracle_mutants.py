"""Planted mistakes: each mutant of the oracle source must fail at least one pin.

Every mutation is applied to a temporary copy of ``oracle/hca_oracle.c``, built
with gcc and bound in place of the real oracle for the duration of one test.
This shows that the pin battery below would notice a dropped term, a wrong
sign, an off-by-one index or a swapped operand in the oracle.  CPU only.
"""
import ctypes
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests._independent import dense_masked_attention, exact_block_mean_bf16, widen

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

MUTANTS = {
    "window_one_short": ("for (int64_t p = lo; p <= t; ++p) {\n                    keys[nk] = k + ",
                         "for (int64_t p = lo + 1; p <= t; ++p) {\n                    keys[nk] = k + "),
    "entry_visible_late": ("if (b * block + block - 1 <= t) {", "if (b * block + block <= t) {"),
    "entry_visible_early": ("if (b * block + block - 1 <= t) {", "if (b * block <= t) {"),
    "gate_sign": ("exp(-widen_bf16(g[d]))", "exp(widen_bf16(g[d]))"),
    "gate_dropped": ("out[d] = (acc / z) * gate;", "out[d] = (acc / z) + 0.0 * gate;"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "values_are_keys": ("acc += s[j] * widen_bf16(vals[j][d]);",
                        "acc += s[j] * widen_bf16(keys[j][d]);"),
    "sum_not_mean": ("round_bf16(s / (double)block)", "round_bf16(s)"),
    "truncating_round": ("nearbyint(ldexp(x, -q))", "trunc(ldexp(x, -q))"),
    "entry_from_keys_only_first_row": ("s += widen_bf16(x[(b * block + i) * ld + d]);",
                                       "s += widen_bf16(x[(b * block) * ld + d]);"),
    "decode_ring_slot": ("keys[nk] = wkb + (p % window) * D;",
                         "keys[nk] = wkb + ((p + 1) % window) * D;"),
    "no_normalisation": ("out[d] = (acc / z) * gate;", "out[d] = acc * gate;"),
}


def _battery():
    """A compact copy of the pins; returns the names of the checks that fail."""
    failures = []

    def check(name, fn):
        try:
            if not fn():
                failures.append(name)
        except Exception:
            failures.append(name)

    # compress against exact rationals
    x = synth.normal_bf16(11, synth.K, (8, 5))

    def compress_exact():
        got = oracle.compress(x, 4)
        want = exact_block_mean_bf16(x, 4)
        return all(Fraction(float(widen(got[b, d]))) == want[b][d]
                   for b in range(2) for d in range(5))
    check("compress_exact", compress_exact)

    # small-block brute force
    T, H, D = 40, 2, 8
    k = synth.normal_bf16(30, synth.K, (T, D))
    v = synth.normal_bf16(30, synth.V, (T, D))
    q = synth.normal_bf16(30, synth.Q, (T, H, D))
    g = synth.normal_bf16(30, synth.G, (T, H, D))

    def brute_small():
        ck, cv = oracle.compress(k, 4), oracle.compress(v, 4)
        got = oracle.attn(q, g, np.arange(T), k, v, 0, ck, cv, block=4, window=4, scale=0.4)
        want = dense_masked_attention(q, g, np.arange(T), k, v, 0, ck, cv, 4, 4, 0.4)
        return np.allclose(got, want, rtol=0, atol=1e-12)
    check("brute_small", brute_small)

    # decode equals the prefill row
    def decode_row():
        ck, cv = oracle.compress(k, 4), oracle.compress(v, 4)
        pre = oracle.attn(q, g, np.arange(T), k, v, 0, ck, cv, block=4, window=4, scale=0.4)
        pos = np.array([0, 3, 4, 9, 39])
        ckb = np.zeros((len(pos), 10, D), np.uint16)
        cvb = np.zeros_like(ckb)
        wk = np.zeros((len(pos), 4, D), np.uint16)
        wv = np.zeros_like(wk)
        for b, t in enumerate(pos):
            n = (t + 1) // 4
            ckb[b, :n], cvb[b, :n] = ck[:n], cv[:n]
            for p in range(max(0, t - 3), t + 1):
                wk[b, p % 4], wv[b, p % 4] = k[p], v[p]
        dec = oracle.decode(q[pos], g[pos], ckb, cvb, wk, wv, pos, block=4, window=4, scale=0.4)
        return np.array_equal(dec, pre[pos])
    check("decode_row", decode_row)

    # row 0 is v0 * sigmoid(g0); G = -inf gives 0
    def row0():
        got = oracle.attn(q[:1], g[:1], [0], k, v, 0, None, None, block=4, window=4)
        return np.allclose(got[0], widen(v[0])[None] / (1 + np.exp(-widen(g[0]))), rtol=1e-15,
                           atol=0)
    check("row0", row0)

    def gate_neg_inf():
        got = oracle.attn(q, np.full(q.shape, 0xFF80, np.uint16), np.arange(T), k, v, 0, None,
                          None, block=4, window=4)
        return np.all(got == 0.0)
    check("gate_neg_inf", gate_neg_inf)

    # bf16 rounding ties to even
    check("round_ties", lambda: oracle.round_bf16(1 + 3 * 2 ** -8) == 0x3F82)
    return failures


@pytest.fixture()
def mutant(tmp_path, request, monkeypatch):
    name = request.param
    src = open(oracle.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path_c = tmp_path / f"{name}.c"
    path_c.write_text(src.replace(old, new, 1))
    path_so = tmp_path / f"{name}.so"
    subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared",
                           "-ffp-contract=off", str(path_c), "-o", str(path_so), "-lm"])
    monkeypatch.setattr(oracle, "_lib", oracle.bind(ctypes.CDLL(str(path_so))))
    return name


def test_battery_passes_on_real_oracle():
    oracle._load()
    assert _battery() == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS), indirect=True)
def test_mutant_is_caught(mutant):
    assert _battery(), f"planted mistake {mutant!r} went unnoticed"
