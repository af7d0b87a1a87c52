"""GPU block compression against the oracle: bit-exact (the kernel sums each
column in binary64 in row order and rounds once, as the oracle does)."""
import numpy as np
import pytest
import torch

import long_context_compressed_hca_amd as hca
import oracle
import synth
from tests.gpu_util import D, dev, gen, host

pytestmark = pytest.mark.gpu


def _compress(k, v):
    T = (k if k is not None else v).shape[0]
    ck = torch.empty((T // 128, D), dtype=torch.bfloat16, device=dev()) if k is not None else None
    cv = torch.empty((T // 128, D), dtype=torch.bfloat16, device=dev()) if v is not None else None
    hca.hca_compress(k, v, ck, cv)
    torch.cuda.synchronize()
    return ck, cv


@pytest.mark.parametrize("T", [128, 300, 2048])
def test_compress_bit_exact(T):
    k, v = gen(1, synth.K, (T, D)), gen(1, synth.V, (T, D))
    ck, cv = _compress(k, v)
    assert np.array_equal(host(ck), oracle.compress(host(k)))
    assert np.array_equal(host(cv), oracle.compress(host(v)))


def test_compress_one_tensor_and_below_one_block():
    k = gen(2, synth.K, (256, D))
    ck, cv = _compress(k, None)
    assert cv is None and np.array_equal(host(ck), oracle.compress(host(k)))
    small = gen(2, synth.V, (100, D))
    ck, cv = _compress(small, small)
    assert ck.shape == (0, D)


def test_compress_strided_rows():
    # rows of a wider buffer: only the first 512 columns are read
    wide = gen(3, synth.K, (384, 1024))
    ck = torch.empty((3, D), dtype=torch.bfloat16, device=dev())
    st = hca.lib().hca_compress(wide.data_ptr(), None, 384, 1024, D, 128, ck.data_ptr(), None,
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert np.array_equal(host(ck), oracle.compress(np.ascontiguousarray(host(wide)[:, :D])))


def test_compress_closed_forms():
    # constant rows -> the constant; an arithmetic progression -> its midpoint (exact)
    c = gen(4, synth.K, (1, D))
    const = c.expand(256, D).contiguous()
    ck, _ = _compress(const, None)
    assert torch.equal(ck, c.expand(2, D))
    i = torch.arange(128, dtype=torch.float32, device=dev())[:, None]
    prog = ((3.0 + 0.25 * i) * torch.ones((1, D), device=dev())).to(torch.bfloat16)
    ck, _ = _compress(prog, None)
    assert torch.all(ck.float() == 3.0 + 0.25 * 127 / 2)


def test_compress_ties_round_to_even():
    # block mean exactly half way between two bf16 neighbours: 1 + 2^-8 -> 1.0,
    # 1 + 3*2^-8 -> 1 + 2^-6.  Rows: 64 copies of a and 64 of b average (a+b)/2.
    def block(a, b):
        x = torch.empty((128, D), dtype=torch.float32, device=dev())
        x[:64], x[64:] = a, b
        return x.to(torch.bfloat16)
    k = torch.cat([block(1.0, 1.0 + 2 ** -7), block(1.0 + 2 ** -7, 1.0 + 2 ** -6)])
    ck, _ = _compress(k, None)
    got = ck.float().cpu().numpy()
    assert np.all(got[0] == 1.0) and np.all(got[1] == 1.0 + 2 ** -6)
    assert np.array_equal(host(ck), oracle.compress(host(k)))


@pytest.mark.parametrize("T", [131072, 1048576])
def test_compress_full_size(T):
    # the 128K prefill's K/V and the whole 1M-token history
    k, v = gen(5, synth.K, (T, D)), gen(5, synth.V, (T, D))
    ck, cv = _compress(k, v)
    assert np.array_equal(host(ck), oracle.compress(host(k)))
    assert np.array_equal(host(cv), oracle.compress(host(v)))


def test_device_generator_matches_host_generator():
    t = gen(9, synth.G, (3, 5, 512))
    assert np.array_equal(host(t), synth.normal_bf16(9, synth.G, (3, 5, 512)))
    big = synth.normal_bf16_device(9, synth.Q, (1 << 20,), dev(), start=123456789)
    assert np.array_equal(host(big)[:1000], synth.normal_bf16(9, synth.Q, 1000, start=123456789))
