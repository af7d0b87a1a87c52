"""Shared pieces of the GPU parity tests: input construction, host copies,
row sampling, and the comparison against the fp64 oracle.

Tolerance (the oracle is exact up to fp64 rounding; the GPU path rounds P to
bf16, accumulates in fp32 and may round the output to bf16):
  relative L2 over the compared outputs <= 1e-2, max |gpu - oracle| <= 3e-2,
  and, so that a bug confined to a few rows cannot hide in the global norm,
  the worst per-(query, head) row relative L2 <= 2e-2.
"""
from __future__ import annotations

import numpy as np

import synth

REL_L2 = 1e-2
MAX_ABS = 3e-2
ROW_REL_L2 = 2e-2
D = 512


def dev():
    import torch
    return torch.device("cuda:0")


def host(t) -> np.ndarray:
    """A device bf16 tensor -> numpy uint16 bit patterns."""
    import torch
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t) -> np.ndarray:
    import torch
    return t.to(torch.float32).cpu().numpy().astype(np.float64)


def gen(seed, tid, shape):
    return synth.normal_bf16_device(seed, tid, shape, dev())


def compare(got: np.ndarray, ref: np.ndarray, what: str = "") -> dict:
    """got/ref: [..., D] float64.  Asserts the tolerance; returns the figures."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    diff = got - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.abs(diff).max()) if diff.size else 0.0
    rows_ref = ref.reshape(-1, ref.shape[-1])
    rows_diff = diff.reshape(-1, ref.shape[-1])
    row_rel = np.linalg.norm(rows_diff, axis=1) / np.maximum(np.linalg.norm(rows_ref, axis=1),
                                                               1e-30)
    worst = float(row_rel.max()) if row_rel.size else 0.0
    figures = dict(rel_l2=rel, max_abs=mx, worst_row_rel_l2=worst,
                   worst_row=int(row_rel.argmax()) if row_rel.size else -1)
    assert rel <= REL_L2 and mx <= MAX_ABS and worst <= ROW_REL_L2, f"{what}: {figures}"
    return figures


def sample_positions(q_start: int, Tq: int, seed: int, n_blocks: int = 32,
                     n_random: int = 256) -> np.ndarray:
    """Query positions to check at full size: the rows around block ends
    (128m-1, 128m, 128m+1) of n_blocks seeded blocks, the first and last four
    queries, and n_random seeded random queries."""
    rng = np.random.default_rng(seed)
    lo, hi = q_start, q_start + Tq - 1
    first_m, last_m = lo // 128 + 1, hi // 128
    picks = set(range(lo, min(lo + 4, hi + 1))) | set(range(max(lo, hi - 3), hi + 1))
    if last_m >= first_m:
        for m in rng.choice(np.arange(first_m, last_m + 1),
                            size=min(n_blocks, last_m - first_m + 1), replace=False):
            picks |= {p for p in (128 * m - 1, 128 * m, 128 * m + 1) if lo <= p <= hi}
    picks |= set(int(x) for x in rng.integers(lo, hi + 1, size=n_random))
    return np.array(sorted(picks), dtype=np.int64)


class Prefill:
    """Seeded inputs of one prefill problem, generated on the GPU.

    Raw K/V rows exist for positions kv_start .. q_start+Tq-1; queries sit at
    q_start .. q_start+Tq-1.  Entries are compressed on the GPU with the
    library's compress (checked bit-exact elsewhere); the oracle recompresses
    the host copy itself."""

    def __init__(self, seed, Tq, H, q_start=0, kv_start=None, out_dtype="bf16",
                 k_total=None):
        import torch
        self.seed, self.Tq, self.H, self.q_start = seed, Tq, H, q_start
        first_needed = max(0, q_start - 127)
        self.kv_start = first_needed if kv_start is None else kv_start
        # K/V are generated for every position 0 .. end so entries can be built
        end = q_start + Tq if k_total is None else k_total
        self.k_all = gen(seed, synth.K, (end, D))
        self.v_all = gen(seed, synth.V, (end, D))
        self.k = self.k_all[self.kv_start:q_start + Tq]
        self.v = self.v_all[self.kv_start:q_start + Tq]
        self.q = gen(seed, synth.Q, (Tq, H, D))
        self.g = gen(seed, synth.G, (Tq, H, D))
        self.Nc = (q_start + Tq) // 128
        self.ck = torch.empty((self.Nc, D), dtype=torch.bfloat16, device=dev())
        self.cv = torch.empty_like(self.ck)
        self.out = torch.empty((Tq, H, D), device=dev(),
                               dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16)

    def run(self, **kw):
        import long_context_compressed_hca_amd as hca
        if self.Nc:
            hca.hca_compress(self.k_all[:self.Nc * 128], self.v_all[:self.Nc * 128], self.ck,
                             self.cv)
        hca.hca_attn_prefill(self.q, self.g, self.k, self.v, self.ck if self.Nc else None,
                             self.cv if self.Nc else None, self.out, q_start=self.q_start,
                             kv_start=self.kv_start, **kw)
        return self.out

    def oracle(self, positions=None, **kw):
        """fp64 oracle rows for the given absolute positions (default: all)."""
        import oracle
        import torch
        if positions is None:
            positions = np.arange(self.q_start, self.q_start + self.Tq)
        idx = torch.as_tensor(positions - self.q_start, device=dev())
        q = host(self.q.index_select(0, idx))
        g = host(self.g.index_select(0, idx))
        k_all, v_all = host(self.k_all), host(self.v_all)
        ck = oracle.compress(k_all[:self.Nc * 128])
        cv = oracle.compress(v_all[:self.Nc * 128])
        return oracle.attn(q, g, positions, k_all[self.kv_start:], v_all[self.kv_start:],
                           self.kv_start, ck, cv, **kw)

    def gpu_rows(self, positions):
        import torch
        idx = torch.as_tensor(positions - self.q_start, device=dev())
        return host_f64(self.out.index_select(0, idx))
