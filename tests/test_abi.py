"""The C ABI library: it loads without a GPU, exports what include/hca.h declares,
and rejects invalid arguments on the host before any HIP call.

Every call here fails validation (or is a documented no-op) before the library
touches the HIP runtime, so fake, never-dereferenced pointer values are safe.
"""
import ctypes
import os
import re
import subprocess

import pytest

import long_context_compressed_hca_amd as hca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED = hca.HCA_OK, hca.HCA_ERR_INVALID_ARG, hca.HCA_ERR_UNSUPPORTED
P = 0x10000          # an aligned fake device address (never dereferenced)
MIS = 0x10008        # not 16-byte aligned


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hca.LIB_PATH):
        from long_context_compressed_hca_amd import _build
        _build.build()
    return hca.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "hca.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hca_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"hca_compress", "hca_attn_prefill", "hca_attn_decode",
            "hca_attn_decode_multi", "hca_attn_prefill_vha"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", hca.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in exported, f"{n} declared in include/hca.h but not exported"
        assert hasattr(L, n)


def test_status_strings(L):
    for st in range(5):
        assert L.hca_status_string(st)
    assert L.hca_version() >= 100


def prefill(L, **kw):
    a = dict(q=P, g=P, k=P, v=P, ck=P, cv=P, Tq=256, q_start=0, Tkv=256, kv_start=0, Nc=2, H=64,
             D=512, block=128, window=128, scale=512 ** -0.5, out=P, dtype=0, stream=None)
    a.update(kw)
    return L.hca_attn_prefill(a["q"], a["g"], a["k"], a["v"], a["ck"], a["cv"], a["Tq"],
                              a["q_start"], a["Tkv"], a["kv_start"], a["Nc"], a["H"], a["D"],
                              a["block"], a["window"], a["scale"], a["out"], a["dtype"],
                              a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(D=256), UNSUPPORTED), (dict(block=64), UNSUPPORTED), (dict(window=256), UNSUPPORTED),
    (dict(H=0), UNSUPPORTED), (dict(H=65), UNSUPPORTED),
    (dict(Tq=-1), INVALID), (dict(q_start=-5), INVALID), (dict(Nc=-1), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=float("inf")), INVALID), (dict(scale=-1.0), INVALID),
    (dict(dtype=7), INVALID),
    # the first query at 300 needs raw rows from 173, but K starts at 200
    (dict(q_start=300, Tq=10, kv_start=200, Tkv=110, Nc=2), INVALID),
    # raw rows end before the last query
    (dict(Tkv=255), INVALID),
    # the last query (position 255) sees entries 0 and 1
    (dict(Nc=1), INVALID),
    (dict(q=0), INVALID), (dict(g=MIS), INVALID), (dict(out=0), INVALID), (dict(ck=0), INVALID),
    (dict(q_start=2 ** 31 - 10, Tq=20, kv_start=2 ** 31 - 200, Tkv=300, Nc=2 ** 24),
     UNSUPPORTED),
])
def test_prefill_rejects(L, kw, status):
    assert prefill(L, **kw) == status
    assert L.hca_last_error()


def test_prefill_noop_and_optional_entries(L):
    assert prefill(L, Tq=0) == OK          # nothing to do, no HIP call
    assert prefill(L, Tq=0, q=0, out=0) == OK
    # no entry is visible below position 127, so ck/cv may be NULL there (still
    # rejected here for another reason: the output pointer is misaligned)
    assert prefill(L, Tq=100, Tkv=100, Nc=0, ck=0, cv=0, out=MIS) == INVALID
    assert b"out" in L.hca_last_error()


def prefill_lse(L, **kw):
    a = dict(q=P, g=P, k=P, v=P, ck=P, cv=P, Tq=256, q_start=0, Tkv=256, kv_start=0, Nc=2, H=64,
             D=512, block=128, window=128, scale=512 ** -0.5, out=P, dtype=0, lse=P, stream=None)
    a.update(kw)
    return L.hca_attn_prefill_lse(a["q"], a["g"], a["k"], a["v"], a["ck"], a["cv"], a["Tq"],
                                  a["q_start"], a["Tkv"], a["kv_start"], a["Nc"], a["H"], a["D"],
                                  a["block"], a["window"], a["scale"], a["out"], a["dtype"],
                                  a["lse"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(lse=0), INVALID), (dict(lse=P + 2), INVALID), (dict(H=65), UNSUPPORTED),
    (dict(dtype=3), INVALID), (dict(Nc=1), INVALID), (dict(q=0), INVALID),
])
def test_prefill_lse_rejects(L, kw, status):
    assert prefill_lse(L, **kw) == status
    assert L.hca_last_error()


def test_prefill_lse_noop(L):
    assert prefill_lse(L, Tq=0, q=0, out=0, lse=0) == OK


def prefill_vha(L, **kw):
    a = dict(q=P, g=P, k=P, v=P, ck=P, cv=P, Tq=256, q_start=0, Tkv=256, kv_start=0, Nc=2, H=64,
             D=512, block=128, window=128, scale=512 ** -0.5, up=P, down=P, rank=8, out=P,
             dtype=0, stream=None)
    a.update(kw)
    return L.hca_attn_prefill_vha(a["q"], a["g"], a["k"], a["v"], a["ck"], a["cv"], a["Tq"],
                                  a["q_start"], a["Tkv"], a["kv_start"], a["Nc"], a["H"], a["D"],
                                  a["block"], a["window"], a["scale"], a["up"], a["down"],
                                  a["rank"], a["out"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(H=32), UNSUPPORTED), (dict(rank=0), UNSUPPORTED), (dict(rank=6), UNSUPPORTED),
    (dict(rank=36), UNSUPPORTED), (dict(rank=-4), UNSUPPORTED), (dict(up=0), INVALID),
    (dict(down=MIS), INVALID), (dict(Nc=1), INVALID), (dict(q=0), INVALID),
    (dict(D=256), UNSUPPORTED),
])
def test_prefill_vha_rejects(L, kw, status):
    assert prefill_vha(L, **kw) == status


def test_prefill_vha_noop(L):
    assert prefill_vha(L, Tq=0, q=0, out=0, up=0, down=0) == OK


def decode(L, **kw):
    a = dict(q=P, g=P, ck=P, cv=P, nc_cap=256, wk=P, wv=P, pos=P, B=64, H=64, D=512, block=128,
             window=128, scale=512 ** -0.5, out=P, dtype=0, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return L.hca_attn_decode(a["q"], a["g"], a["ck"], a["cv"], a["nc_cap"], a["wk"], a["wv"],
                             a["pos"], a["B"], a["H"], a["D"], a["block"], a["window"],
                             a["scale"], a["out"], a["dtype"], a["ws"], a["ws_bytes"],
                             a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(D=128), UNSUPPORTED), (dict(H=0), UNSUPPORTED), (dict(H=80), UNSUPPORTED),
    (dict(nc_cap=(1 << 24) + 1), UNSUPPORTED), (dict(B=-1), INVALID),
    (dict(nc_cap=-1), INVALID),
    (dict(pos=0), INVALID), (dict(pos=P + 4), INVALID), (dict(wk=0), INVALID),
    (dict(ck=0), INVALID), (dict(scale=float("nan")), INVALID), (dict(dtype=3), INVALID),
])
def test_decode_rejects(L, kw, status):
    assert decode(L, **kw) == status


WORKSPACE = hca.HCA_ERR_WORKSPACE


def test_decode_workspace_size(L):
    # batches that fill the GPU need none; small ones split their keys across
    # workgroups and need fp32 partials (32 + 16 * 512 floats per 16 heads and split)
    assert L.hca_decode_workspace_size(64, 64, 512, 256) == 0
    assert L.hca_decode_workspace_size(256, 16, 512, 4096) == 0
    small = L.hca_decode_workspace_size(8, 64, 512, 256)
    assert small > 0 and small % ((32 + 16 * 512) * 4 * 8 * 4) == 0
    assert L.hca_decode_workspace_size(1, 8, 512, 1 << 20) > 0
    assert L.hca_decode_workspace_size(1, 8, 512, 0) == 0   # 8 window tiles: no split
    for bad in [(0, 64, 512, 256), (8, 65, 512, 256), (8, 64, 256, 256), (8, 64, 512, -1)]:
        assert L.hca_decode_workspace_size(*bad) == 0


def decode_noalloc(L, **kw):
    a = dict(q=P, g=P, ck=P, cv=P, nc_cap=256, wk=P, wv=P, pos=P, B=64, H=64, D=512, block=128,
             window=128, scale=512 ** -0.5, out=P, dtype=0, stream=None)
    a.update(kw)
    return L.hca_attn_decode_noalloc(a["q"], a["g"], a["ck"], a["cv"], a["nc_cap"], a["wk"],
                                     a["wv"], a["pos"], a["B"], a["H"], a["D"], a["block"],
                                     a["window"], a["scale"], a["out"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(D=128), UNSUPPORTED), (dict(H=0), UNSUPPORTED), (dict(B=-1), INVALID),
    (dict(pos=0), INVALID), (dict(q=MIS), INVALID), (dict(scale=-1.0), INVALID),
])
def test_decode_noalloc_rejects(L, kw, status):
    assert decode_noalloc(L, **kw) == status
    assert decode_noalloc(L, B=0) == OK


def test_decode_workspace_errors(L):
    need = L.hca_decode_workspace_size(8, 64, 512, 256)
    assert decode(L, B=8, ws=None, ws_bytes=0) == WORKSPACE
    assert decode(L, B=8, ws=P, ws_bytes=need - 1) == WORKSPACE
    assert decode(L, B=8, ws=MIS, ws_bytes=need) == INVALID
    assert "workspace" in L.hca_last_error().decode()


def test_decode_noop(L):
    assert decode(L, B=0) == OK


def decode_multi(L, **kw):
    a = dict(q=P, g=P, ck=P, cv=P, nc_cap=256, wk=P, wv=P, nk=P, nv=P, pos=P, B=64, M=3, H=64,
             D=512, block=128, window=128, scale=512 ** -0.5, out=P, dtype=0, stream=None)
    a.update(kw)
    return L.hca_attn_decode_multi(a["q"], a["g"], a["ck"], a["cv"], a["nc_cap"], a["wk"],
                                   a["wv"], a["nk"], a["nv"], a["pos"], a["B"], a["M"], a["H"],
                                   a["D"], a["block"], a["window"], a["scale"], a["out"],
                                   a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(D=128), UNSUPPORTED), (dict(M=0), UNSUPPORTED), (dict(M=17), UNSUPPORTED),
    (dict(H=0), UNSUPPORTED), (dict(M=16, H=80), UNSUPPORTED),
    (dict(M=1, H=128), UNSUPPORTED), (dict(M=8, H=128), UNSUPPORTED),
    (dict(B=-1), INVALID), (dict(nc_cap=-1), INVALID), (dict(pos=0), INVALID),
    (dict(pos=P + 4), INVALID), (dict(nk=0), INVALID), (dict(nv=MIS), INVALID),
    (dict(ck=0), INVALID), (dict(scale=0.0), INVALID), (dict(dtype=2), INVALID),
])
def test_decode_multi_rejects(L, kw, status):
    assert decode_multi(L, **kw) == status


def test_decode_multi_noop(L):
    assert decode_multi(L, B=0) == OK


def backward(L, **kw):
    a = dict(q=P, g=P, k=P, v=P, ck=P, cv=P, dout=P, T=1000, H=64, D=512, block=128, window=128,
             scale=512 ** -0.5, dq=P, dk=P, dv=P, dg=P, ws=P, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return L.hca_attn_backward(a["q"], a["g"], a["k"], a["v"], a["ck"], a["cv"], a["dout"],
                               a["T"], a["H"], a["D"], a["block"], a["window"], a["scale"],
                               a["dq"], a["dk"], a["dv"], a["dg"], a["ws"], a["ws_bytes"],
                               a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(D=256), UNSUPPORTED), (dict(block=64), UNSUPPORTED), (dict(window=256), UNSUPPORTED),
    (dict(H=0), UNSUPPORTED), (dict(H=65), UNSUPPORTED), (dict(T=1 << 26), UNSUPPORTED),
    (dict(T=-1), INVALID), (dict(scale=float("inf")), INVALID), (dict(q=0), INVALID),
    (dict(dout=MIS), INVALID), (dict(dg=0), INVALID), (dict(ck=0), INVALID),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=1000), WORKSPACE), (dict(ws=MIS), INVALID),
])
def test_backward_rejects(L, kw, status):
    assert backward(L, **kw) == status


def test_backward_noop_and_optional_entries(L):
    assert backward(L, T=0, q=0, ws=None, ws_bytes=0) == OK
    # below one block there are no entries: ck, cv may be NULL (rejected later for
    # the missing workspace, so nothing is launched)
    assert backward(L, T=100, ck=0, cv=0, ws=None, ws_bytes=0) == WORKSPACE


def backward_saved(L, **kw):
    a = dict(q=P, g=P, k=P, v=P, ck=P, cv=P, out=P, dtype=0, lse=P, dout=P, T=1000, H=64, D=512,
             block=128, window=128, scale=512 ** -0.5, dq=P, dk=P, dv=P, dg=P, ws=P,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return L.hca_attn_backward_saved(a["q"], a["g"], a["k"], a["v"], a["ck"], a["cv"], a["out"],
                                     a["dtype"], a["lse"], a["dout"], a["T"], a["H"], a["D"],
                                     a["block"], a["window"], a["scale"], a["dq"], a["dk"],
                                     a["dv"], a["dg"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(out=0), INVALID), (dict(out=MIS), INVALID), (dict(lse=0), INVALID),
    (dict(lse=P + 2), INVALID), (dict(dtype=2), INVALID), (dict(H=65), UNSUPPORTED),
    (dict(T=-1), INVALID), (dict(ck=0), INVALID), (dict(ws=None), WORKSPACE),
    (dict(ws_bytes=1000), WORKSPACE),
])
def test_backward_saved_rejects(L, kw, status):
    assert backward_saved(L, **kw) == status


def test_backward_saved_noop(L):
    assert backward_saved(L, T=0, q=0, out=0, lse=0, ws=None, ws_bytes=0) == OK


def test_backward_workspace_size(L):
    # per query row 2 floats + 512 bf16 of dA, per entry 2 x 512 floats, each
    # array 256-byte aligned, plus 256 bytes of alignment slack
    up = lambda x: (x + 255) // 256 * 256
    for T, H in [(1, 1), (1000, 64), (131072, 64), (257, 3)]:
        rows, nc = T * H, T // 128
        want = 2 * up(4 * rows) + up(1024 * rows) + 2 * up(2048 * nc) + 256
        assert L.hca_backward_workspace_size(T, H, 512) == want
    for bad in [(0, 64, 512), (100, 0, 512), (100, 65, 512), (100, 8, 256), (1 << 26, 64, 512)]:
        assert L.hca_backward_workspace_size(*bad) == 0


def compress(L, k=P, v=P, T=256, ld=512, D=512, block=128, ck=P, cv=P):
    return L.hca_compress(k, v, T, ld, D, block, ck, cv, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=256), UNSUPPORTED), (dict(block=32), UNSUPPORTED), (dict(T=-1), INVALID),
    (dict(ld=500), INVALID), (dict(ld=516), INVALID), (dict(k=0), INVALID),
    (dict(cv=0), INVALID), (dict(k=0, ck=0, v=0, cv=0), INVALID), (dict(k=MIS), INVALID),
])
def test_compress_rejects(L, kw, status):
    assert compress(L, **kw) == status


def test_compress_noop_below_one_block(L):
    assert compress(L, T=127) == OK
    assert compress(L, T=0) == OK
    assert compress(L, T=100, ck=0, cv=0) == OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(hca, "_lib", None)
    monkeypatch.setattr(hca, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        hca.lib()


def gate(L, **kw):
    a = dict(latent=P, w=P, T=256, R=1024, N=32768, g=P, stream=None)
    a.update(kw)
    return L.hca_gate_logits(a["latent"], a["w"], a["T"], a["R"], a["N"], a["g"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(R=32), UNSUPPORTED), (dict(R=96), UNSUPPORTED), (dict(R=0), UNSUPPORTED),
    (dict(R=16384 + 64), UNSUPPORTED), (dict(N=1024), UNSUPPORTED), (dict(N=3072), UNSUPPORTED),
    (dict(N=65536 + 2048), UNSUPPORTED), (dict(T=-1), INVALID), (dict(latent=0), INVALID),
    (dict(w=0), INVALID), (dict(g=0), INVALID),
])
def test_gate_logits_rejects(L, kw, status):
    assert gate(L, **kw) == status


def test_gate_logits_noop(L):
    assert gate(L, T=0, latent=0, w=0, g=0) == OK
