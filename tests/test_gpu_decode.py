"""GPU decode attention against the fp64 oracle (every output compared)."""
import numpy as np
import pytest
import torch

import long_context_compressed_hca_amd as hca
import oracle
import synth
from tests.gpu_util import D, Prefill, compare, dev, gen, host, host_f64

pytestmark = pytest.mark.gpu


class Decode:
    def __init__(self, seed, positions, H=64, nc_cap=None, out_dtype="bf16"):
        positions = np.asarray(positions, dtype=np.int64)
        B = len(positions)
        self.nc_cap = int(max((positions + 1) // 128)) if nc_cap is None else nc_cap
        self.q = gen(seed, synth.Q, (B, H, D))
        self.g = gen(seed, synth.G, (B, H, D))
        self.ck = gen(seed, synth.CK, (B, self.nc_cap, D))
        self.cv = gen(seed, synth.CV, (B, self.nc_cap, D))
        self.wk = gen(seed, synth.WK, (B, 128, D))
        self.wv = gen(seed, synth.WV, (B, 128, D))
        self.pos_np = positions
        self.pos = torch.as_tensor(positions, device=dev())
        self.out = torch.empty((B, H, D), device=dev(),
                               dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16)

    def run(self):
        hca.hca_attn_decode(self.q, self.g, self.ck, self.cv, self.wk, self.wv, self.pos,
                            self.out)
        torch.cuda.synchronize()
        return self.out

    def oracle(self):
        return oracle.decode(host(self.q), host(self.g), host(self.ck), host(self.cv),
                             host(self.wk), host(self.wv), self.pos_np)


def test_64_sequences_32k_history():
    # the batched decode workload: 64 sequences, new token at 32768,
    # 256 entries + 128 window rows each, 64 heads
    d = Decode(seed=4, positions=[32768] * 64, nc_cap=256)
    print(compare(host_f64(d.run()), d.oracle(), "decode B=64"))


@pytest.mark.parametrize("H", [1, 8, 16, 24, 32, 48, 64])
def test_mixed_positions(H):
    positions = [0, 1, 5, 126, 127, 128, 129, 255, 256, 383, 1000, 4095, 4096, 32767]
    d = Decode(seed=10 + H, positions=positions, H=H, out_dtype="f32")
    compare(host_f64(d.run()), d.oracle(), f"decode H={H}")


@pytest.mark.parametrize("B", [128, 256])
def test_large_batches(B):
    # 64 heads: 128 sequences take 32 heads per workgroup, 256 take all 64
    rng = np.random.default_rng(B)
    positions = rng.integers(0, 3000, size=B)
    positions[:4] = [0, 127, 128, 2999]
    d = Decode(seed=17 + B, positions=positions, H=64, out_dtype="f32")
    compare(host_f64(d.run()), d.oracle(), f"decode B={B}")


@pytest.mark.parametrize("B,H,pos", [(1, 64, 20000), (2, 8, 70000), (8, 64, 32768),
                                     (3, 40, 30000), (16, 16, 20000)])
def test_small_batches_split_keys(B, H, pos):
    # batches too small to fill the GPU split each sequence's keys across
    # workgroups and merge the partial states through the workspace
    import long_context_compressed_hca_amd as h
    rng = np.random.default_rng(B * 1000 + H)
    positions = rng.integers(0, pos + 1, size=B)
    positions[0] = pos
    if B > 1:
        positions[-1] = min(positions[-1], 5)  # a sequence with fewer tiles than streams
    d = Decode(seed=18 + B + H, positions=positions, H=H, out_dtype="f32")
    need = h.decode_workspace_size(B, H, d.nc_cap)
    assert need > 0
    ws = torch.full((need,), 255, dtype=torch.uint8, device=dev())  # stale contents
    hca.hca_attn_decode(d.q, d.g, d.ck, d.cv, d.wk, d.wv, d.pos, d.out, workspace=ws)
    torch.cuda.synchronize()
    first = d.out.clone()
    compare(host_f64(first), d.oracle(), f"split decode B={B} H={H}")
    hca.hca_attn_decode(d.q, d.g, d.ck, d.cv, d.wk, d.wv, d.pos, d.out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(first, d.out)  # same workspace again: same bits


def test_cache_larger_than_needed():
    d = Decode(seed=12, positions=[200, 700, 50], H=32, nc_cap=40)
    compare(host_f64(d.run()), d.oracle(), "nc_cap 40")


def test_gate_limits():
    d = Decode(seed=13, positions=[10, 300, 5000], H=16, out_dtype="f32")
    d.g = torch.full_like(d.g, float("-inf"))
    assert torch.all(d.run() == 0)
    d.g = torch.zeros_like(d.g)
    half = d.run().clone()
    d.g = torch.full_like(d.g, float("inf"))
    assert torch.equal(2 * half, d.run())


def test_decode_matches_prefill_row():
    # decode at position t reads the same keys as row t of a prefill over [0, t]
    T, H = 1000, 64
    p = Prefill(seed=14, Tq=T, H=H, out_dtype="f32")
    p.run()
    positions = np.array([0, 127, 128, 640, 999])
    d = Decode(seed=14, positions=positions, H=H, nc_cap=T // 128, out_dtype="f32")
    for b, t in enumerate(positions):
        d.q[b], d.g[b] = p.q[t], p.g[t]
        n = (t + 1) // 128
        d.ck[b, :n], d.cv[b, :n] = p.ck[:n], p.cv[:n]
        for s in range(max(0, t - 127), t + 1):
            d.wk[b, s % 128], d.wv[b, s % 128] = p.k_all[s], p.v_all[s]
    got = d.run()
    torch.cuda.synchronize()
    torch.testing.assert_close(got, p.out[torch.as_tensor(positions, device=dev())],
                               rtol=2e-2, atol=2e-3)
    compare(host_f64(got), d.oracle(), "decode rows")


def test_unused_ring_slots_and_cache_rows_are_never_read():
    # ring slots past the new token (t < 127) and cache rows past the visible
    # entries may hold anything, NaN included
    positions = [0, 5, 100, 126, 127, 300, 1100]
    d = Decode(seed=16, positions=positions, H=64, nc_cap=12, out_dtype="f32")
    for b, t in enumerate(positions):
        if t < 127:
            d.wk[b, t + 1:], d.wv[b, t + 1:] = float("nan"), float("nan")
        n = (t + 1) // 128
        d.ck[b, n:], d.cv[b, n:] = float("nan"), float("nan")
    got = host_f64(d.run())
    assert np.isfinite(got).all()
    compare(got, d.oracle(), "NaN in unused rows")


def test_batch_zero_is_noop():
    d = Decode(seed=15, positions=[5], H=16)
    hca.hca_attn_decode(d.q[:0], d.g[:0], d.ck[:0], d.cv[:0], d.wk[:0], d.wv[:0], d.pos[:0],
                        d.out[:0])


def test_entry_cache_of_2_21_entries():
    # 2^21 entries per sequence (a token past position 2^28): entry offsets no
    # longer fit one 32-bit buffer descriptor, and the per-tile-descriptor
    # kernel takes the batch.  The last entry's key is head 0's query times 4
    # (exact in bf16), so at scale 1/sqrt(512) its score is about 90 while the
    # others stay near N(0, 1): head 0's output is close to that entry's value
    # times the gate, and an entry read from a wrapped offset would show.  The
    # score also rises far above the first tile's maximum, so the exact-maximum
    # second pass runs.
    nc = 1 << 21
    pos = (nc << 7) + 5
    d = Decode(seed=30, positions=[pos], H=64, nc_cap=nc, out_dtype="f32")
    d.ck[0, nc - 1] = d.q[0, 0] * 4
    torch.cuda.synchronize()
    got = host_f64(d.run())
    print(compare(got, d.oracle(), "decode with 2^21 entries"))
    g0 = host_f64(d.g[0, 0])
    want = host_f64(d.cv[0, nc - 1]) / (1.0 + np.exp(-g0))
    assert np.abs(got[0, 0] - want).max() <= 3e-2
