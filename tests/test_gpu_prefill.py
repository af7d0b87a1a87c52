"""GPU prefill attention against the fp64 oracle.

Small and medium problems are compared in full (every row, several tiles and
a ragged tail of rows); the full-size workloads (T = 8192 and 128K with 64
heads, and the last 64K-query chunk of a 1M-token sequence) are compared on
sampled rows (block ends, first/last queries, random rows) with every head.
"""
import numpy as np
import pytest
import torch

import long_context_compressed_hca_amd as hca
from tests.gpu_util import Prefill, compare, host_f64, sample_positions

pytestmark = pytest.mark.gpu


def _full_check(p: Prefill, what: str):
    p.run()
    torch.cuda.synchronize()
    return compare(host_f64(p.out), p.oracle(), what)


def test_2048_tokens_8_heads_f32_out():
    # the small workload: T = 2048, H = 8, fp32 output
    p = Prefill(seed=1, Tq=2048, H=8, out_dtype="f32")
    print(_full_check(p, "T=2048 H=8 f32"))


@pytest.mark.parametrize("Tq,H", [(1, 64), (5, 8), (127, 16), (128, 64), (129, 8), (300, 64),
                                  (700, 24), (1000, 1), (450, 3), (260, 40)])
def test_small_shapes(Tq, H):
    p = Prefill(seed=100 + Tq + H, Tq=Tq, H=H)
    _full_check(p, f"Tq={Tq} H={H}")


@pytest.mark.parametrize("q_start,Tq,H", [(300, 400, 64), (1000, 129, 8), (255, 2, 64),
                                          (128, 256, 16)])
def test_chunk_with_history(q_start, Tq, H):
    # queries from q_start, raw rows from the first one the window needs,
    # entries for every completed block before the chunk's end
    p = Prefill(seed=7 + q_start, Tq=Tq, H=H, q_start=q_start)
    _full_check(p, f"chunk q_start={q_start}")


def test_chunk_equals_monolithic_bitwise():
    # a chunk aligned to the workgroup's 128 rows computes the same tiles in
    # the same order as the monolithic call
    full = Prefill(seed=21, Tq=1024, H=64)
    full.run()
    a = 512
    part = Prefill(seed=21, Tq=1024 - a, H=64, q_start=a)
    part.q, part.g = full.q[a:], full.g[a:]
    part.run()
    torch.cuda.synchronize()
    assert torch.equal(part.out, full.out[a:])


def test_gate_limits():
    p = Prefill(seed=31, Tq=300, H=16, out_dtype="f32")
    p.g = torch.full_like(p.g, float("-inf"))
    p.run()
    torch.cuda.synchronize()
    assert torch.all(p.out == 0)                       # sigmoid(-inf) = 0 exactly
    p.g = torch.zeros_like(p.g)
    half = p.run().clone()
    p.g = torch.full_like(p.g, float("inf"))
    whole = p.run().clone()
    torch.cuda.synchronize()
    assert torch.equal(2 * half, whole)                # sigmoid(0) = 1/2, sigmoid(inf) = 1
    compare(host_f64(whole), p.oracle(), "G=+inf")


def test_constant_values():
    p = Prefill(seed=41, Tq=600, H=8, out_dtype="f32")
    c = p.v_all[:1].clone()
    p.v_all.copy_(c.expand_as(p.v_all))
    p.run()
    torch.cuda.synchronize()
    want = c.float()[None] * torch.sigmoid(p.g.float())
    torch.testing.assert_close(p.out, want, rtol=1e-4, atol=1e-6)


def test_scale_power_of_two_is_exact():
    # (2Q, scale/2) gives bitwise the same result as (Q, scale)
    p = Prefill(seed=51, Tq=400, H=16, out_dtype="f32")
    ref = p.run().clone()
    p.q = (p.q.float() * 2).to(torch.bfloat16)
    twice = p.run(scale=512 ** -0.5 / 2).clone()
    torch.cuda.synchronize()
    assert torch.equal(ref, twice)


def test_noop_and_errors():
    p = Prefill(seed=61, Tq=256, H=8)
    with pytest.raises(hca.HcaError):     # kv_start past the first query's window
        hca.hca_attn_prefill(p.q[200:], p.g[200:], p.k[150:], p.v[150:], p.ck, p.cv,
                             p.out[200:], q_start=200, kv_start=150)


def _sampled(p: Prefill, seed: int, what: str, **kw):
    pos = sample_positions(p.q_start, p.Tq, seed, **kw)
    p.run()
    torch.cuda.synchronize()
    fig = compare(p.gpu_rows(pos), p.oracle(pos), what)
    print(what, len(pos), "positions", fig)


def test_8192_tokens_64_heads_sampled():
    _sampled(Prefill(seed=2, Tq=8192, H=64), 2, "T=8192 H=64")


def test_128k_tokens_64_heads_sampled():
    _sampled(Prefill(seed=3, Tq=131072, H=64), 3, "T=131072 H=64")


def test_1m_context_last_chunk_sampled():
    # the last 65536 queries of a 1,048,576-token sequence: 8192 entries of history
    T = 1 << 20
    p = Prefill(seed=5, Tq=65536, H=64, q_start=T - 65536, k_total=T)
    assert p.kv_start == T - 65536 - 127 and p.Nc == 8192
    _sampled(p, 5, "1M chunk")
