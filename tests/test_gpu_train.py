"""The training pair on the GPU: prefill that keeps each row's log-sum-exp
(hca_attn_prefill_lse) and the backward pass from that saved state
(hca_attn_backward_saved), against the fp64 oracle.

* lse: the kernel sums the bf16-rounded weights exp(x - m) (relative error at
  most 2^-9 each) in fp32, so |lse - oracle| <= ln(1 + 2^-8) = 3.9e-3 covers the
  rounding with room for the fp32 score and sum errors.  The output is bitwise
  that of hca_attn_prefill.
* Backward from a given state: the state is the oracle's (its gated output
  rounded to bf16 or kept in f32, its lse in f32), the GPU backward and the
  oracle's saved-state routine take the same values, so the differences are the
  kernels' roundings (weights, dA and score gradients to bf16, fp32 sums); the
  bounds and floors of the recompute backward's tests apply, with dq and dk held
  row by row against the oracle with dA rounded to bf16 (given Dt, the score
  gradients no longer sum to zero exactly, so a row whose gradients nearly
  cancel moves with the rounding of dA) and tensor-wide against the exact one.
* End to end (GPU prefill_lse, then the GPU backward): against the exact
  gradients, tensor-wide bounds (the bf16 output's rounding enters
  Dt = <dO, out>, relative 2^-9 per element, which moves rows whose score
  gradients nearly cancel by more than 2e-2 of themselves)."""
import numpy as np
import pytest
import torch

import long_context_compressed_hca_amd as hca
import oracle
import synth
from tests.gpu_util import D, Prefill, dev, host, host_f64, sample_positions
from tests.test_gpu_backward import Backward, _compare

pytestmark = pytest.mark.gpu
LSE_TOL = float(np.log1p(2.0 ** -8))


def _lse_case(p):
    lse = torch.full((p.Tq, p.H), float("nan"), dtype=torch.float32, device=dev())
    ref_out = p.run().clone()
    p.out.fill_(float("nan"))
    hca.hca_attn_prefill_lse(p.q, p.g, p.k, p.v, p.ck if p.Nc else None,
                             p.cv if p.Nc else None, p.out, lse, q_start=p.q_start,
                             kv_start=p.kv_start)
    torch.cuda.synchronize()
    assert torch.equal(p.out.view(torch.uint8), ref_out.view(torch.uint8)), "output differs"
    pos = np.arange(p.q_start, p.q_start + p.Tq)
    kh = host(p.k_all)
    want = oracle.attn_lse(host(p.q), pos, kh[p.kv_start:], p.kv_start,
                           oracle.compress(kh[:p.Nc * 128]))
    got = lse.cpu().numpy().astype(np.float64)
    err = float(np.abs(got - want).max())
    print(f"lse Tq={p.Tq} H={p.H} q_start={p.q_start}: max |err| {err:.3g}", flush=True)
    assert np.all(np.isfinite(got)) and err <= LSE_TOL, err


@pytest.mark.parametrize("Tq,H,q_start,out_dtype", [
    (600, 8, 0, "f32"), (300, 64, 0, "bf16"), (257, 64, 900, "bf16"), (1, 1, 0, "bf16"),
    (129, 5, 0, "f32"), (700, 16, 3000, "bf16"),
])
def test_prefill_lse(Tq, H, q_start, out_dtype):
    print(f"prefill_lse Tq={Tq} H={H} q_start={q_start} {out_dtype}", flush=True)
    _lse_case(Prefill(seed=500 + Tq + H, Tq=Tq, H=H, q_start=q_start, out_dtype=out_dtype))


def test_prefill_lse_peaked_rows():
    # rows aimed at late window keys take the exact-maximum rerun; lse must come
    # from that pass's reference
    from tests.test_gpu_peaked import _peaked_prefill
    p, n_over = _peaked_prefill(95, 300, 64, 0, "bf16")
    assert n_over > 1000
    _lse_case(p)


class Saved(Backward):
    """A backward problem whose forward state is the oracle's."""

    def state(self, out_dtype):
        q, g, k, v = host(self.q), host(self.g), host(self.k), host(self.v)
        pos = np.arange(self.T)
        ck, cv = oracle.compress(k), oracle.compress(v)
        o = oracle.attn(q, g, pos, k, v, 0, ck, cv, nthreads=8)
        lse = oracle.attn_lse(q, pos, k, 0, ck, nthreads=8)
        lse_f32 = lse.astype(np.float32)
        if out_dtype == "bf16":
            bits = synth.f64_to_bf16_bits(o)
            self.out = torch.from_numpy(bits.view(np.int16)).to(dev()).view(torch.bfloat16)
            self.o_used = synth.bf16_bits_to_f32(bits).astype(np.float64)
        else:
            o32 = o.astype(np.float32)
            self.out = torch.from_numpy(o32).to(dev())
            self.o_used = o32.astype(np.float64)
        self.lse = torch.from_numpy(lse_f32).to(dev())
        self.lse_used = lse_f32.astype(np.float64)

    def run_saved(self, workspace=None):
        if self.Nc:
            hca.hca_compress(self.k[:self.Nc * 128], self.v[:self.Nc * 128], self.ck, self.cv)
        hca.hca_attn_backward_saved(self.q, self.g, self.k, self.v, self.ck if self.Nc else None,
                                    self.cv if self.Nc else None, self.out, self.lse, self.do,
                                    self.dq, self.dk, self.dv, self.dg, workspace=workspace)
        torch.cuda.synchronize()

    def check_saved(self):
        args = (host(self.q), host(self.g), host(self.do), self.o_used, self.lse_used,
                host(self.k), host(self.v))
        exact = oracle.attn_backward_saved(*args, nthreads=8)
        rounded = oracle.attn_backward_saved(*args, round_da=True, nthreads=8)
        got = [t.cpu().numpy().astype(np.float64) for t in (self.dq, self.dk, self.dv, self.dg)]
        figs = {n: _compare(a, b, n) for n, a, b in zip(("dq", "dk", "dv", "dg"), got, exact)}
        for n, a, b in zip(("dq~", "dk~", "dv~"), got, rounded):
            figs[n] = _compare(a, b, n)
        print(f"saved T={self.T} H={self.H}", figs, flush=True)
        # the weights' and Dt's rounding-free reference for dq, dk is the oracle
        # with dA rounded as the kernels round it, every row; against the exact
        # one, tensor-wide only, and not at T = 1, where the one row's score
        # gradient is a rounding residue (p = 1: dp - Dt vanishes but for the
        # roundings of dA and of the given output)
        need = [("dv", None), ("dg", None), ("dq~", None), ("dk~", None), ("dv~", None)]
        if self.T > 1:
            need += [("dq", ("rel_l2_ok", "max_rel_ok")), ("dk", ("rel_l2_ok", "max_rel_ok"))]
        bad = [n for n, only in need
               if not (figs[n]["ok"] if only is None else all(figs[n][c] for c in only))]
        assert not bad, f"saved T={self.T} H={self.H}: {bad} {figs}"


@pytest.mark.parametrize("T,H,out_dtype", [(600, 8, "bf16"), (300, 64, "f32"), (100, 3, "bf16"),
                                           (1, 1, "f32"), (129, 5, "bf16"), (1000, 16, "bf16")])
def test_backward_saved_against_oracle(T, H, out_dtype):
    print(f"backward_saved T={T} H={H} {out_dtype}", flush=True)
    b = Saved(2000 + T + H, T, H)
    b.state(out_dtype)
    b.run_saved()
    b.check_saved()


def test_backward_saved_entry_chunks_and_workspace():
    print("backward_saved T=4500 H=2", flush=True)
    b = Saved(78, 4500, 2)
    b.state("bf16")
    ws = torch.empty(hca.backward_workspace_size(4500, 2), dtype=torch.uint8, device=dev())
    ws.fill_(0xFF)
    b.run_saved(workspace=ws)
    b.check_saved()


def _end_to_end(T, H, seed, out_dtype):
    b = Backward(seed, T, H)
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out = torch.empty((T, H, D), dtype=dt, device=dev())
    lse = torch.empty((T, H), dtype=torch.float32, device=dev())
    if b.Nc:
        hca.hca_compress(b.k[:b.Nc * 128], b.v[:b.Nc * 128], b.ck, b.cv)
    ck, cv = (b.ck, b.cv) if b.Nc else (None, None)
    hca.hca_attn_prefill_lse(b.q, b.g, b.k, b.v, ck, cv, out, lse)
    hca.hca_attn_backward_saved(b.q, b.g, b.k, b.v, ck, cv, out, lse, b.do, b.dq, b.dk, b.dv,
                                b.dg)
    torch.cuda.synchronize()
    return b


@pytest.mark.parametrize("T,H,out_dtype", [(600, 8, "bf16"), (1000, 16, "bf16"),
                                           (300, 64, "f32")])
def test_training_pair_end_to_end(T, H, out_dtype):
    print(f"prefill_lse + backward_saved T={T} H={H} {out_dtype}", flush=True)
    b = _end_to_end(T, H, 3000 + T, out_dtype)
    want = b.oracle()
    got = [t.cpu().numpy().astype(np.float64) for t in (b.dq, b.dk, b.dv, b.dg)]
    figs = {n: _compare(a, w, n) for n, a, w in zip(("dq", "dk", "dv", "dg"), got, want)}
    print(figs, flush=True)
    assert all(f["rel_l2_ok"] and f["max_rel_ok"] for f in figs.values()), figs


def test_training_pair_128k_sampled_rows_and_sums():
    """128K x 64 heads through both GPU calls: sampled rows of dq and dg against
    the exact gradients (tensor-wide bounds over the sample), and the key-gradient
    sums the mathematics fixes (sum dk = 0, sum dv = sum dO sigmoid(g)) within 1e-2
    of the summed magnitudes."""
    T, H = 131072, 64
    print(f"prefill_lse + backward_saved T={T} H={H} (sampled rows)", flush=True)
    b = _end_to_end(T, H, 129, "bf16")
    pos = sample_positions(0, T, 129, n_blocks=8, n_random=24)
    idx = torch.as_tensor(pos, device=dev())
    qs, gs, dos = (host(t.index_select(0, idx)) for t in (b.q, b.g, b.do))
    dq_e, dg_e = oracle.attn_backward_rows(qs, gs, dos, pos, host(b.k), host(b.v), nthreads=16)
    f_dq = _compare(b.dq.index_select(0, idx).cpu().numpy().astype(np.float64), dq_e, "dq")
    f_dg = _compare(b.dg.index_select(0, idx).cpu().numpy().astype(np.float64), dg_e, "dg")
    print(len(pos), "positions", {"dq": f_dq, "dg": f_dg}, flush=True)
    assert f_dq["rel_l2_ok"] and f_dq["max_rel_ok"] and f_dg["ok"], (f_dq, f_dg)
    want_v = torch.zeros(D, dtype=torch.float64, device=dev())
    for t0 in range(0, T, 8192):
        sl = slice(t0, min(T, t0 + 8192))
        want_v += (b.do[sl].double() * torch.sigmoid(b.g[sl].double())).sum(dim=(0, 1))
    for name, t, want in (("dv", b.dv, want_v), ("dk", b.dk, torch.zeros_like(want_v))):
        s = t.double().sum(dim=0)
        worst = float(((s - want).abs() / t.double().abs().sum(dim=0)).max())
        print(f"sum of {name}: worst dim error / magnitude {worst:.3g}", flush=True)
        assert worst <= 1e-2, (name, worst)
