"""hca_attn_decode_noalloc (the decode entry point for callers that cannot
allocate) against hca_attn_decode with a caller-owned workspace: two calls in a
row on batches that split their keys across workgroups (so the built-in scratch
is used), the second smaller than the first.  The kernels are the same, so the
outputs must be equal bit for bit; both are also held to the oracle's tolerance."""
import numpy as np
import pytest
import torch

import long_context_compressed_hca_amd as hca
from tests.gpu_util import compare, dev, host_f64
from tests.test_gpu_decode import Decode

pytestmark = pytest.mark.gpu


def _check(d, what):
    B, H = d.q.shape[0], d.q.shape[1]
    need = hca.decode_workspace_size(B, H, d.nc_cap)
    assert 0 < need <= 8421376, need  # split batch, within the built-in scratch
    ws = torch.full((need,), 255, dtype=torch.uint8, device=dev())
    ref = torch.empty_like(d.out)
    hca.hca_attn_decode(d.q, d.g, d.ck, d.cv, d.wk, d.wv, d.pos, ref, workspace=ws)
    got = torch.full_like(d.out, float("nan"))
    hca.hca_attn_decode_noalloc(d.q, d.g, d.ck, d.cv, d.wk, d.wv, d.pos, got)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), what
    compare(host_f64(got), d.oracle(), what)


def test_noalloc_matches_workspace_entry_point():
    rng = np.random.default_rng(77)
    big = Decode(seed=77, positions=rng.integers(20000, 40000, size=16), H=64, out_dtype="f32")
    _check(big, "noalloc B=16 H=64")
    small = Decode(seed=78, positions=[30000, 129, 7], H=40, out_dtype="bf16")
    _check(small, "noalloc B=3 H=40 (after a larger call)")
