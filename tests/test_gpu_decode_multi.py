"""GPU multi-token decode (M new tokens per sequence) against the fp64 oracle,
every output compared."""
import numpy as np
import pytest
import torch

import long_context_compressed_hca_amd as hca
import oracle
import synth
from tests.gpu_util import D, compare, dev, gen, host, host_f64

pytestmark = pytest.mark.gpu


class DecodeMulti:
    def __init__(self, seed, positions, M, H=64, nc_cap=None, out_dtype="bf16"):
        positions = np.asarray(positions, dtype=np.int64)
        B = len(positions)
        self.nc_cap = int(max((positions + M) // 128)) if nc_cap is None else nc_cap
        self.q = gen(seed, synth.Q, (B, M, H, D))
        self.g = gen(seed, synth.G, (B, M, H, D))
        self.ck = gen(seed, synth.CK, (B, self.nc_cap, D))
        self.cv = gen(seed, synth.CV, (B, self.nc_cap, D))
        self.wk = gen(seed, synth.WK, (B, 128, D))
        self.wv = gen(seed, synth.WV, (B, 128, D))
        self.nk = gen(seed, synth.NK, (B, M, D))
        self.nv = gen(seed, synth.NV, (B, M, D))
        self.pos_np = positions
        self.pos = torch.as_tensor(positions, device=dev())
        self.out = torch.empty((B, M, H, D), device=dev(),
                               dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16)

    def run(self):
        hca.hca_attn_decode_multi(self.q, self.g, self.ck, self.cv, self.wk, self.wv, self.nk,
                                  self.nv, self.pos, self.out)
        torch.cuda.synchronize()
        return self.out

    def oracle(self):
        return oracle.decode_multi(host(self.q), host(self.g), host(self.ck), host(self.cv),
                                   host(self.wk), host(self.wv), host(self.nk), host(self.nv),
                                   self.pos_np)


def test_verify_64_sequences_32k_history():
    # the verify step of two-token drafts: 64 sequences, 3 new tokens at
    # 32765 .. 32767 (the last one completes block 255), 64 heads
    d = DecodeMulti(seed=5, positions=[32765] * 64, M=3, nc_cap=256)
    print(compare(host_f64(d.run()), d.oracle(), "decode_multi B=64 M=3"))


POSITIONS = [0, 1, 5, 124, 125, 126, 127, 128, 129, 253, 254, 255, 256, 383, 1000, 4093]


@pytest.mark.parametrize("M,H", [(1, 64), (2, 16), (3, 64), (4, 32), (8, 64), (16, 16), (3, 8),
                                 (2, 24), (5, 1)])
def test_mixed_positions(M, H):
    d = DecodeMulti(seed=20 + M + H, positions=POSITIONS, M=M, H=H, out_dtype="f32")
    compare(host_f64(d.run()), d.oracle(), f"decode_multi M={M} H={H}")


@pytest.mark.parametrize("B,M", [(16, 3), (64, 2), (64, 3), (64, 4)])
def test_batch_sizes(B, M):
    # H = 64: 4M blocks of 16 rows per sequence; these batches take 1, 2, 3 and
    # 4 blocks per workgroup
    rng = np.random.default_rng(B + M)
    positions = rng.integers(0, 3000, size=B)
    positions[:5] = [0, 126, 127, 128, 2999]
    d = DecodeMulti(seed=30 + B + M, positions=positions, M=M, out_dtype="f32")
    compare(host_f64(d.run()), d.oracle(), f"decode_multi B={B} M={M}")


def test_one_token_equals_decode():
    # M = 1 with the new row in nk/nv is single-token decode with the row in its
    # ring slot: both against the oracle
    positions = [0, 127, 128, 700, 4095]
    d = DecodeMulti(seed=40, positions=positions, M=1, H=32, out_dtype="f32")
    got = host_f64(d.run())[:, 0]
    wk, wv = d.wk.clone(), d.wv.clone()
    for b, t in enumerate(positions):
        wk[b, t % 128], wv[b, t % 128] = d.nk[b, 0], d.nv[b, 0]
    out = torch.empty((len(positions), 32, D), device=dev(), dtype=torch.float32)
    hca.hca_attn_decode(d.q[:, 0].contiguous(), d.g[:, 0].contiguous(), d.ck, d.cv, wk, wv,
                        d.pos, out)
    torch.cuda.synchronize()
    ref = oracle.decode(host(d.q[:, 0].contiguous()), host(d.g[:, 0].contiguous()), host(d.ck),
                        host(d.cv), host(wk), host(wv), d.pos_np)
    compare(got, ref, "M=1 multi")
    compare(host_f64(out), ref, "M=1 single")


def test_unread_slots_and_entries_may_hold_nan():
    # the ring slot of position pos-128 (overwritten by the first new token once
    # committed), entries past floor((pos+M)/128) and nothing else may be NaN
    positions = [130, 300, 1021, 5000]
    M = 3
    d = DecodeMulti(seed=41, positions=positions, M=M, H=16, nc_cap=48, out_dtype="f32")
    nan = float("nan")
    for b, t in enumerate(positions):
        d.wk[b, t % 128] = nan
        d.wv[b, t % 128] = nan
        d.ck[b, (t + M) // 128:] = nan
        d.cv[b, (t + M) // 128:] = nan
    got = host_f64(d.run())
    assert np.isfinite(got).all()
    compare(got, d.oracle(), "NaN in unread rows")


def test_bf16_output_and_repeat_calls():
    d = DecodeMulti(seed=42, positions=[40, 2000, 9000], M=3, H=64)
    first = d.run().clone()
    assert torch.equal(first, d.run())
    compare(host_f64(first), d.oracle(), "bf16 out")


def test_largest_row_count_per_sequence():
    # M * H = 1024 rows per sequence (16 tokens x 64 heads), positions around
    # block ends and t = 0
    d = DecodeMulti(seed=43, positions=[0, 112, 240, 5000], M=16, H=64, out_dtype="f32")
    compare(host_f64(d.run()), d.oracle(), "decode_multi M=16 H=64")


def test_empty_batch_is_noop():
    d = DecodeMulti(seed=44, positions=[5], M=2, H=16)
    e = lambda t: t[:0]
    hca.hca_attn_decode_multi(e(d.q), e(d.g), e(d.ck), e(d.cv), e(d.wk), e(d.wv), e(d.nk),
                              e(d.nv), e(d.pos), e(d.out))
    torch.cuda.synchronize()
