"""GPU gate logits of the low-rank gate (hca_gate_logits) and the low-rank gated
prefill (gate logits, then prefill) against the fp64 oracle.

Inputs: latent ~ N(0,1) and W_g ~ N(0,1)/32 in bf16 (so G ~ N(0,1), the scale of
the stored-logit workloads), R = 1024 (the 4096-wide hidden state / 4).  The
kernel accumulates in fp32 and rounds G to bf16 once: each logit is checked
against the exact value within 2^-8 relative plus 2e-3 absolute (the fp32
accumulation of 1024 products), and exactly where inputs make every partial
sum exact."""
import numpy as np
import pytest
import torch

import long_context_compressed_hca_amd as hca
import oracle
import synth
from tests.gpu_util import Prefill, compare, dev, gen, host, host_f64, sample_positions

pytestmark = pytest.mark.gpu
LAT, WG = 10, 11   # synth tensor ids of the latent and the gate weight


def _inputs(seed, T, R, N):
    lat = gen(seed, LAT, (T, R))
    w = (gen(seed, WG, (N, R)) * (1.0 / 32)).contiguous()   # exact power-of-two scaling
    return lat, w


def _check_logits(got_bits, want):
    got = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    err = np.abs(got - want)
    bound = 2.0 ** -8 * np.abs(want) + 2e-3
    assert np.all(err <= bound), float((err - bound).max())


@pytest.mark.parametrize("T,N", [(300, 4096), (1, 2048), (257, 8192), (1024, 32768)])
def test_logits_against_oracle(T, N):
    R = 1024
    lat, w = _inputs(100 + T, T, R, N)
    g = torch.empty((T, N), dtype=torch.bfloat16, device=dev())
    hca.hca_gate_logits(lat, w, g)
    torch.cuda.synchronize()
    _check_logits(host(g), oracle.gate_logits(host(lat), host(w)))


def test_logits_large_sampled_rows():
    # 4133 queries x 64 heads x 512 (17 t tiles, the last one ragged; several
    # tiles per workgroup): the first, boundary and last rows and sampled rows
    T, R, N = 4133, 1024, 32768
    lat, w = _inputs(7, T, R, N)
    g = torch.empty((T, N), dtype=torch.bfloat16, device=dev())
    hca.hca_gate_logits(lat, w, g)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(250, 262), np.arange(4090, 4100), np.arange(T - 8, T),
                                     np.random.default_rng(7).integers(0, T, 64)]))
    idx = torch.as_tensor(rows, device=dev())
    want = oracle.gate_logits(host(lat.index_select(0, idx)), host(w))
    _check_logits(host(g.index_select(0, idx)), want)


@pytest.mark.parametrize("T,R,N", [
    (300, 64, 2048),      # one tile per workgroup, one K step per tile
    (2085, 64, 16384),    # two tiles per workgroup with one K step each, ragged last t tile
    (4096, 128, 16384),   # several tiles per workgroup, two K steps each
    (1100, 192, 32768),   # three K steps per tile (the W_g buffers wrap mid-tile)
])
def test_logits_exact_when_partial_sums_are_exact(T, R, N):
    # integer latent, weights multiples of 1/8: every fp32 partial sum is exact
    # (multiples of 1/8 below 2^21), so the GPU's result is the exact value
    # rounded to nearest-even bf16, bit for bit, whatever the order of the sums
    rng = np.random.default_rng(3 + R + T)
    lat_f = rng.integers(-2, 3, size=(T, R)).astype(np.float32)
    w_f = (rng.integers(-4, 5, size=(N, R)) / 8).astype(np.float32)
    lat_b, w_b = synth.f32_to_bf16_bits(lat_f), synth.f32_to_bf16_bits(w_f)
    to_dev = lambda b: torch.from_numpy(b.view(np.int16)).to(dev()).view(torch.bfloat16)
    g = torch.empty((T, N), dtype=torch.bfloat16, device=dev())
    hca.hca_gate_logits(to_dev(lat_b), to_dev(w_b), g)
    torch.cuda.synchronize()
    want = oracle.gate_logits(lat_b, w_b)
    assert np.all(np.abs(want) < 2.0 ** 21)
    np.testing.assert_array_equal(host(g), synth.f32_to_bf16_bits(want.astype(np.float32)))


@pytest.mark.parametrize("T,H,q_start", [(600, 8, 0), (300, 64, 0), (257, 16, 1000)])
def test_lowrank_gated_prefill(T, H, q_start):
    R = 1024
    p = Prefill(seed=110 + H, Tq=T, H=H, q_start=q_start, out_dtype="f32")
    lat, w = _inputs(110 + H, T, R, H * 512)
    if p.Nc:
        hca.hca_compress(p.k_all[:p.Nc * 128], p.v_all[:p.Nc * 128], p.ck, p.cv)
    hca.hca_attn_prefill_lowrank_gate(p.q, lat, w, p.k, p.v, p.ck if p.Nc else None,
                                      p.cv if p.Nc else None, p.out, q_start=q_start,
                                      kv_start=p.kv_start)
    torch.cuda.synchronize()
    ka, va = host(p.k_all), host(p.v_all)
    ck, cv = oracle.compress(ka[:p.Nc * 128]), oracle.compress(va[:p.Nc * 128])
    want = oracle.attn_lowrank_gate(host(p.q), host(lat), host(w), q_start + np.arange(T),
                                    ka[p.kv_start:], va[p.kv_start:], p.kv_start, ck, cv)
    compare(host_f64(p.out), want, f"low-rank gated prefill T={T} H={H}")


def test_empty_is_noop():
    lat, w = _inputs(1, 4, 64, 2048)
    g = torch.empty((0, 2048), dtype=torch.bfloat16, device=dev())
    hca.hca_gate_logits(lat[:0], w, g)


def test_logits_128k_sampled_rows():
    # the measured shape, 131072 x 1024 x 32768: the GEMM at full size, rows of
    # seeded tiles (the first, last and random ones, every n) against the oracle
    T, R, N = 131072, 1024, 32768
    lat, w = _inputs(31, T, R, N)
    g = torch.empty((T, N), dtype=torch.bfloat16, device=dev())
    hca.hca_gate_logits(lat, w, g)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([np.arange(0, 4), np.arange(T - 4, T), np.arange(255, 259),
                                     rng.integers(0, T, 48)]))
    idx = torch.as_tensor(rows, device=dev())
    want = oracle.gate_logits(host(lat.index_select(0, idx)), host(w))
    _check_logits(host(g.index_select(0, idx)), want)
