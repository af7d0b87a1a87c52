"""GPU backward pass (hca_attn_backward) against the fp64 oracle's gradients.

Whole sequences at positions 0 .. T-1: q, g, dout ~ N(0,1) bf16, k, v ~ N(0,1)
bf16, entries compressed on the GPU by the library's compress (bit-exact with the
oracle's elsewhere).  The kernels round the softmax weights, the score
gradients and dA = dout * sigmoid(g) to bf16 for the products and accumulate in
fp32, so each gradient is held to the forward's relative bounds: relative L2 over
the tensor <= 1e-2, worst row relative L2 <= 2e-2, and max |gpu - oracle| <= 3e-2
times the largest |oracle| element of the tensor (gradients are not O(1) like the
forward's output, so the absolute bound is taken relative to their scale).  Rows
far smaller than the tensor's median row, and gradients that vanish exactly, are
held to a floor (1e-3 of the median row norm; 1e-5 per element)."""
import numpy as np
import pytest
import torch

import long_context_compressed_hca_amd as hca
import oracle
import synth
from tests.gpu_util import D, dev, gen, host

pytestmark = pytest.mark.gpu
DOUT = 12  # synth tensor id of the upstream gradient

REL_L2, ROW_REL_L2, MAX_REL = 1e-2, 2e-2, 3e-2
ATOL = 1e-5  # fp32 rounding of O(1) sums; far below bf16 resolution of the inputs


def _compare(got, ref, what):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    diff = got - ref
    # norms below ATOL per element count as zero: a gradient that vanishes exactly
    # (a query with one visible key has dq = 0) is met to fp32 rounding, not
    # relative to itself
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), ATOL * np.sqrt(ref.size)))
    rows_ref = ref.reshape(-1, D)
    rows_diff = diff.reshape(-1, D)
    nref = np.linalg.norm(rows_ref, axis=1)
    # rows whose gradient is tiny next to the tensor's typical row (a key no
    # query weighs) are held to the tensor's scale instead of their own
    floor = max(1e-3 * float(np.median(nref)), ATOL * np.sqrt(D)) if nref.size else 1.0
    row_rel = np.linalg.norm(rows_diff, axis=1) / np.maximum(nref, floor)
    mx = float(np.abs(diff).max())
    scale = max(float(np.abs(ref).max()), ATOL / MAX_REL)
    fig = dict(rel_l2=rel, worst_row_rel_l2=float(row_rel.max()), max_abs=mx, ref_max=scale,
               worst_row=int(row_rel.argmax()))
    fig["rel_l2_ok"] = rel <= REL_L2
    fig["max_rel_ok"] = mx <= MAX_REL * scale
    fig["ok"] = fig["rel_l2_ok"] and fig["max_rel_ok"] and fig["worst_row_rel_l2"] <= ROW_REL_L2
    return fig


class Backward:
    def __init__(self, seed, T, H):
        self.T, self.H = T, H
        self.q = gen(seed, synth.Q, (T, H, D))
        self.g = gen(seed, synth.G, (T, H, D))
        self.do = gen(seed, DOUT, (T, H, D))
        self.k = gen(seed, synth.K, (T, D))
        self.v = gen(seed, synth.V, (T, D))
        self.Nc = T // 128
        self.ck = torch.empty((self.Nc, D), dtype=torch.bfloat16, device=dev())
        self.cv = torch.empty_like(self.ck)
        f32 = dict(dtype=torch.float32, device=dev())
        self.dq = torch.full((T, H, D), float("nan"), **f32)
        self.dg = torch.full((T, H, D), float("nan"), **f32)
        self.dk = torch.full((T, D), float("nan"), **f32)
        self.dv = torch.full((T, D), float("nan"), **f32)

    def run(self, workspace=None):
        if self.Nc:
            hca.hca_compress(self.k[:self.Nc * 128], self.v[:self.Nc * 128], self.ck, self.cv)
        hca.hca_attn_backward(self.q, self.g, self.k, self.v, self.ck if self.Nc else None,
                              self.cv if self.Nc else None, self.do, self.dq, self.dk, self.dv,
                              self.dg, workspace=workspace)
        torch.cuda.synchronize()

    def oracle(self):
        return oracle.attn_backward(host(self.q), host(self.g), host(self.do), host(self.k),
                                    host(self.v), nthreads=8)

    def oracle_rounded_da(self):
        """Oracle gradients of q, k, v for dA = dout * sigmoid(g) rounded to bf16, the
        operand the kernels multiply: the oracle is called with that dA as the
        upstream gradient and a gate of logit 40, whose sigmoid is exactly 1 in
        fp64 (exp(-40) < 2^-53)."""
        g = synth.bf16_bits_to_f32(host(self.g)).astype(np.float64)
        do = synth.bf16_bits_to_f32(host(self.do)).astype(np.float64)
        da = synth.f64_to_bf16_bits(do / (1.0 + np.exp(-g)))
        ones = np.full(da.shape, 0x4220, dtype=np.uint16)  # bf16 40.0
        return oracle.attn_backward(host(self.q), ones, da, host(self.k), host(self.v),
                                    nthreads=8)[:3]

    def check(self):
        """Against the exact gradients: every tensor within the relative bounds, and
        every row of dk, dv and dg.  Rows of dq are checked against the gradients
        for the bf16-rounded dA: a query whose score gradients nearly cancel (one
        dominant key; dq is then far below its terms) has a dq that the rounding
        of dA moves by more than 2e-2 of itself, as it would any bf16 attention
        backward."""
        dq, dk, dv, dg = self.oracle()
        got = [t.cpu().numpy().astype(np.float64) for t in (self.dq, self.dk, self.dv, self.dg)]
        figs = {name: _compare(a, b, name)
                for name, a, b in zip(("dq", "dk", "dv", "dg"), got, (dq, dk, dv, dg))}
        dq_r, dk_r, dv_r = self.oracle_rounded_da()
        for name, a, b in zip(("dq~", "dk~", "dv~"), got, (dq_r, dk_r, dv_r)):
            figs[name] = _compare(a, b, name)
        need = [("dq", ("rel_l2_ok", "max_rel_ok")), ("dk", None), ("dv", None), ("dg", None),
                ("dq~", None), ("dk~", None), ("dv~", None)]
        print(f"T={self.T} H={self.H}", figs, flush=True)
        bad = [n for n, only in need
               if not (figs[n]["ok"] if only is None else all(figs[n][c] for c in only))]
        assert not bad, f"T={self.T} H={self.H}: {bad} {figs}"
        return figs


@pytest.mark.parametrize("T,H", [(600, 8), (300, 64), (100, 3), (1, 1), (129, 5), (1000, 16)])
def test_backward_against_oracle(T, H):
    print(f"backward T={T} H={H}", flush=True)
    b = Backward(1000 + T + H, T, H)
    b.run()
    b.check()


def test_backward_entry_chunks():
    # past 4096 queries an entry's queries are split over several tasks whose
    # contributions are added atomically
    print("backward T=4500 H=2", flush=True)
    b = Backward(77, 4500, 2)
    b.run()
    b.check()


def test_backward_workspace_reused():
    # a workspace holding another call's data (and a smaller call after a larger
    # one) gives the same gradients
    ws = torch.empty(hca.backward_workspace_size(700, 16), dtype=torch.uint8, device=dev())
    big = Backward(5, 700, 16)
    big.run(workspace=ws)
    small = Backward(6, 300, 8)
    small.run(workspace=ws)
    small.check()
    again = [t.clone() for t in (big.dq, big.dk, big.dv, big.dg)]
    big.run(workspace=ws)
    for a, b in zip(again[::3], (big.dq, big.dg)):
        assert torch.equal(a, b)  # row-wise gradients are deterministic
    big.check()


def test_backward_empty():
    e = torch.empty((0, 4, D), dtype=torch.bfloat16, device=dev())
    kv = torch.empty((0, D), dtype=torch.bfloat16, device=dev())
    f = torch.empty((0, 4, D), dtype=torch.float32, device=dev())
    fk = torch.empty((0, D), dtype=torch.float32, device=dev())
    hca.hca_attn_backward(e, e, kv, kv, None, None, e, f, fk, fk.clone(), f.clone())
    torch.cuda.synchronize()


def _sums_and_rows(T, seed, n_blocks, n_random):
    """Full-size backward: every row of dq and dg at sampled positions against the
    oracle's per-row routine (dg exact, dq with the bf16-rounded dA, see check()),
    and over the whole sequence the key-gradient sums, which the mathematics fixes:
    sum_t dk[t] = 0 (the score gradients of each row sum to zero) and
    sum_t dv[t] = sum_(t,h) dO sigmoid(g) (the weights of each row sum to one),
    each dim within 1e-2 of the sum of the magnitudes it adds."""
    from tests.gpu_util import sample_positions
    H = 64
    print(f"backward T={T} H={H} (sampled rows)", flush=True)
    b = Backward(seed, T, H)
    b.run()
    pos = sample_positions(0, T, seed, n_blocks=n_blocks, n_random=n_random)
    idx = torch.as_tensor(pos, device=dev())
    qs, gs, dos = (host(t.index_select(0, idx)) for t in (b.q, b.g, b.do))
    kh, vh = host(b.k), host(b.v)
    dq_e, dg_e = oracle.attn_backward_rows(qs, gs, dos, pos, kh, vh, nthreads=16)
    gf = synth.bf16_bits_to_f32(gs).astype(np.float64)
    dof = synth.bf16_bits_to_f32(dos).astype(np.float64)
    da = synth.f64_to_bf16_bits(dof / (1.0 + np.exp(-gf)))
    dq_r, _ = oracle.attn_backward_rows(qs, np.full(da.shape, 0x4220, np.uint16), da, pos, kh, vh,
                                        nthreads=16)
    got_dq = b.dq.index_select(0, idx).cpu().numpy().astype(np.float64)
    got_dg = b.dg.index_select(0, idx).cpu().numpy().astype(np.float64)
    f_dq, f_dg = _compare(got_dq, dq_r, "dq~"), _compare(got_dg, dg_e, "dg")
    print(len(pos), "positions", {"dq~": f_dq, "dg": f_dg}, flush=True)
    assert f_dq["ok"] and f_dg["ok"], (f_dq, f_dg)
    # the sums over the whole sequence (fp64 on the GPU, from the inputs)
    want_v = torch.zeros(D, dtype=torch.float64, device=dev())
    for t0 in range(0, T, 8192):
        sl = slice(t0, min(T, t0 + 8192))
        want_v += (b.do[sl].double() * torch.sigmoid(b.g[sl].double())).sum(dim=(0, 1))
    for name, t, want in (("dv", b.dv, want_v), ("dk", b.dk, torch.zeros_like(want_v))):
        s = t.double().sum(dim=0)
        mag = t.double().abs().sum(dim=0)
        worst = float(((s - want).abs() / mag).max())
        print(f"sum of {name}: worst dim error / magnitude {worst:.3g}", flush=True)
        assert worst <= 1e-2, (name, worst)


def test_backward_8k_sampled_rows_and_sums():
    _sums_and_rows(8192, 88, n_blocks=16, n_random=64)


def test_backward_128k_sampled_rows_and_sums():
    _sums_and_rows(131072, 128, n_blocks=8, n_random=24)
