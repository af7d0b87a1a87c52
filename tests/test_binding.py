"""The Python binding's own checks (CPU only): every tensor's shape is compared
with the query's before any pointer reaches the C ABI, which cannot see sizes.

CPU tensors are used: a call with consistent shapes gets as far as the device
check and raises TypeError; a call with one inconsistent shape raises
ValueError before that.
"""
import pytest
import torch

import long_context_compressed_hca_amd as hca

bf = torch.bfloat16
D = 512


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def prefill_args(Tq=4, H=2, Tkv=4, Nc=0):
    return dict(q=z(Tq, H, D), g=z(Tq, H, D), k=z(Tkv, D), v=z(Tkv, D),
                ck=z(Nc, D) if Nc else None, cv=z(Nc, D) if Nc else None,
                out=z(Tq, H, D))


def decode_args(B=3, H=16, nc=2):
    return dict(q=z(B, H, D), g=z(B, H, D), ck=z(B, nc, D), cv=z(B, nc, D),
                wk=z(B, 128, D), wv=z(B, 128, D), pos=z(B, dtype=torch.int64),
                out=z(B, H, D))


def multi_args(B=3, M=2, H=16, nc=2):
    return dict(q=z(B, M, H, D), g=z(B, M, H, D), ck=z(B, nc, D), cv=z(B, nc, D),
                wk=z(B, 128, D), wv=z(B, 128, D), nk=z(B, M, D), nv=z(B, M, D),
                pos=z(B, dtype=torch.int64), out=z(B, M, H, D))


def test_prefill_consistent_shapes_reach_device_check():
    with pytest.raises(TypeError):
        hca.hca_attn_prefill(**prefill_args())
    with pytest.raises(TypeError):
        hca.hca_attn_prefill(**prefill_args(Nc=1, Tkv=200, Tq=200))


@pytest.mark.parametrize("name,bad", [
    ("g", z(4, 2, D + 8)), ("out", z(5, 2, D)), ("k", z(4, D // 2)), ("v", z(3, D)),
    ("ck", z(1, D)), ("cv", z(3, D)),
])
def test_prefill_bad_shapes(name, bad):
    a = prefill_args(Nc=2)
    a[name] = bad
    with pytest.raises(ValueError):
        hca.hca_attn_prefill(**a)


def test_prefill_ck_without_cv():
    a = prefill_args(Nc=1)
    a["cv"] = None
    with pytest.raises(ValueError):
        hca.hca_attn_prefill(**a)


def test_vha_factor_shapes():
    a = prefill_args(H=64)
    with pytest.raises(ValueError):
        hca.hca_attn_prefill_vha(up=z(64, 8), down=z(4, 64), **a)
    with pytest.raises(TypeError):
        hca.hca_attn_prefill_vha(up=z(64, 8), down=z(8, 64), **a)


def test_decode_consistent_shapes_reach_device_check():
    with pytest.raises(TypeError):
        hca.hca_attn_decode(**decode_args())
    a = decode_args()
    a["ck"] = a["cv"] = None  # no cache entries: nc_cap = 0
    with pytest.raises(TypeError):
        hca.hca_attn_decode(**a)


@pytest.mark.parametrize("name,bad", [
    ("g", z(3, 16, 256)), ("out", z(2, 16, D)), ("ck", z(2, 2, D)), ("cv", z(3, 3, D)),
    ("wk", z(3, 64, D)), ("wv", z(3, 128, 256)), ("pos", z(4, dtype=torch.int64)),
])
def test_decode_bad_shapes(name, bad):
    a = decode_args()
    a[name] = bad
    with pytest.raises(ValueError):
        hca.hca_attn_decode(**a)


def test_decode_multi_consistent_shapes_reach_device_check():
    with pytest.raises(TypeError):
        hca.hca_attn_decode_multi(**multi_args())


@pytest.mark.parametrize("name,bad", [
    ("g", z(3, 2, 8, D)), ("out", z(3, 1, 16, D)), ("nk", z(3, 3, D)), ("nv", z(2, 2, D)),
    ("ck", z(3, 2, 256)), ("wk", z(3, 127, D)), ("pos", z(2, dtype=torch.int64)),
])
def test_decode_multi_bad_shapes(name, bad):
    a = multi_args()
    a[name] = bad
    with pytest.raises(ValueError):
        hca.hca_attn_decode_multi(**a)


def test_compress_shapes():
    with pytest.raises(TypeError):
        hca.hca_compress(z(256, D), z(256, D), z(2, D), z(2, D))
    with pytest.raises(ValueError):
        hca.hca_compress(z(256, D), z(256, D), z(1, D), z(2, D))
    with pytest.raises(ValueError):
        hca.hca_compress(z(256, D), z(128, D), z(2, D), z(2, D))
    with pytest.raises(ValueError):
        hca.hca_compress(z(256, D), None, z(2, D), z(2, D))
    with pytest.raises(ValueError):
        hca.hca_compress(None, None, None, None)
