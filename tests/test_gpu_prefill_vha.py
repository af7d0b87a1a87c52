"""GPU prefill with the fused VHA head mix (H = 64) against the fp64 oracle
(attention, gate, then the mix), plus exact identities against plain prefill."""
import numpy as np
import pytest
import torch

import long_context_compressed_hca_amd as hca
import oracle
import synth
from tests.gpu_util import Prefill, compare, dev, gen, host, host_f64, sample_positions

pytestmark = pytest.mark.gpu
H = 64


def _factors(seed, rank):
    # N(0,1) / 8, exact in bf16: the mix is of the same order as the identity
    up = gen(seed, synth.CK, (H, rank)) * 0.125
    down = gen(seed, synth.CV, (rank, H)) * 0.125
    return up.contiguous(), down.contiguous()


def _run_vha(p, up, down):
    if p.Nc:
        hca.hca_compress(p.k_all[:p.Nc * 128], p.v_all[:p.Nc * 128], p.ck, p.cv)
    hca.hca_attn_prefill_vha(p.q, p.g, p.k, p.v, p.ck if p.Nc else None,
                             p.cv if p.Nc else None, up, down, p.out, q_start=p.q_start,
                             kv_start=p.kv_start)
    torch.cuda.synchronize()
    return p.out


@pytest.mark.parametrize("Tq,q_start,rank,out_dtype", [
    (301, 0, 8, "f32"),      # the last item holds one query
    (256, 0, 32, "bf16"),
    (129, 700, 4, "f32"),    # a chunk with history
    (600, 1000, 16, "bf16"),
])
def test_against_oracle(Tq, q_start, rank, out_dtype):
    p = Prefill(seed=60 + rank, Tq=Tq, H=H, q_start=q_start, out_dtype=out_dtype)
    up, down = _factors(60 + rank, rank)
    got = host_f64(_run_vha(p, up, down))
    want = oracle.vha(p.oracle(), host(up), host(down))
    compare(got, want, f"prefill+VHA Tq={Tq} rank={rank}")


def test_zero_up_is_plain_prefill_bitwise():
    for out_dtype in ("f32", "bf16"):
        p = Prefill(seed=70, Tq=259, H=H, q_start=64, out_dtype=out_dtype)
        plain = p.run().clone()
        torch.cuda.synchronize()
        up, down = _factors(70, 8)
        got = _run_vha(p, torch.zeros_like(up), down)
        assert torch.equal(got, plain), out_dtype


@pytest.mark.parametrize("i,j,k,rank", [(5, 40, 0, 8), (40, 5, 7, 8), (63, 0, 31, 32),
                                        (17, 30, 12, 16), (33, 33, 3, 4)])
def test_single_entries_add_one_head(i, j, k, rank):
    # up[:, k] = e_i, down[k, :] = e_j: head i gains bf16(head j); every other head is
    # unchanged bit for bit.  The sum is the MFMA's fp32 accumulate, which is not
    # rounded like an IEEE add: within one fp32 ulp.
    p = Prefill(seed=71, Tq=130, H=H, q_start=200, out_dtype="f32")
    x = p.run().clone()
    torch.cuda.synchronize()
    up = torch.zeros((H, rank), dtype=torch.bfloat16, device=dev())
    down = torch.zeros((rank, H), dtype=torch.bfloat16, device=dev())
    up[i, k] = 1.0
    down[k, j] = 1.0
    got = _run_vha(p, up, down)
    want = x.clone()
    want[:, i] = x[:, i] + x[:, j].to(torch.bfloat16).to(torch.float32)
    others = [h for h in range(H) if h != i]
    assert torch.equal(got[:, others], want[:, others])
    ulp = torch.abs(want[:, i]) * 2.0 ** -23 + 1e-30
    assert torch.all(torch.abs(got[:, i] - want[:, i]) <= ulp)


def test_8192_tokens_sampled():
    p = Prefill(seed=72, Tq=8192, H=H)
    up, down = _factors(72, 8)
    _run_vha(p, up, down)
    pos = sample_positions(0, 8192, 72)
    want = oracle.vha(p.oracle(pos), host(up), host(down))
    compare(p.gpu_rows(pos), want, "prefill+VHA T=8192 sampled")


def test_128k_tokens_sampled():
    p = Prefill(seed=73, Tq=131072, H=H)
    up, down = _factors(73, 8)
    _run_vha(p, up, down)
    pos = sample_positions(0, 131072, 73)
    want = oracle.vha(p.oracle(pos), host(up), host(down))
    compare(p.gpu_rows(pos), want, "prefill+VHA T=131072 sampled")


@pytest.mark.parametrize("Tq,q_start", [(1, 0), (1, 4095), (2, 130), (3, 127)])
def test_few_queries(Tq, q_start):
    # one query (the item's second half empty), two (one full item), three
    p = Prefill(seed=74 + Tq, Tq=Tq, H=H, q_start=q_start, out_dtype="f32")
    up, down = _factors(74, 4)
    got = host_f64(_run_vha(p, up, down))
    want = oracle.vha(p.oracle(), host(up), host(down))
    compare(got, want, f"prefill+VHA Tq={Tq} q_start={q_start}")
