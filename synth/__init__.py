"""Seeded synthetic inputs for HCA: bfloat16 samples of N(0, 1).

This module is shared by both sides of every parity check (the fp64 oracle and
the HIP library).  It holds none of the attention method's arithmetic: it only
turns (seed, tensor id, element index) into a bfloat16 bit pattern.

Generator (counter based, so any element can be produced alone, by any number
of threads, on the host or on the device, with identical bits):

* ``mix64`` is the SplitMix64 output function of Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators" (OOPSLA 2014), with
  increment gamma = 0x9E3779B97F4A7C15.
* The stream key of a tensor is ``mix64((seed << 8) | tensor_id)``.
* Element ``i`` draws ``u = mix64(key + (i + 1) * gamma)`` (all mod 2^64) and
  keeps its top 20 bits as an index into a table of 2^20 normal quantiles:
  ``TABLE[k] = bf16(Phi^-1((k + 0.5) / 2^20))`` (inverse-transform sampling;
  rounding to nearest-even bfloat16).  The values are N(0, 1) as bfloat16,
  truncated at |x| <= 4.9 (probability mass beyond it is 1e-6).

Only integer arithmetic and one table lookup happen per element, so the host
(numpy) and device (``synth_device.hip``) paths agree bit for bit; no libm
call is involved in the per-element path.

Tensor ids used by the HCA workloads: Q=0, K=1, V=2, G=3, CK=4, CV=5, WK=6, WV=7,
NK=8, NV=9 (the new rows of a multi-token decode).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1
TABLE_BITS = 20

Q, K, V, G, CK, CV, WK, WV, NK, NV = range(10)

HERE = os.path.dirname(os.path.abspath(__file__))
DEV_SRC = os.path.join(HERE, "synth_device.hip")
DEV_LIB = os.path.join(HERE, "libhca_synth.so")


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (reference for the vector form)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tensor_id: int) -> int:
    return mix64_int(((seed & 0xFFFFFFFFFFFFFF) << 8) | (tensor_id & 0xFF))


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even); returns uint16 bits.
    Used only to build the quantile table."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, nearest-even (exact for inputs already on the bf16 grid)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


_TABLE = None


def table() -> np.ndarray:
    """The 2^20-entry quantile table (uint16 bfloat16 bits)."""
    global _TABLE
    if _TABLE is None:
        from scipy.special import ndtri
        n = 1 << TABLE_BITS
        p = (np.arange(n, dtype=np.float64) + 0.5) / n
        _TABLE = f64_to_bf16_bits(ndtri(p))
        _TABLE.setflags(write=False)
    return _TABLE


def normal_bf16(seed: int, tensor_id: int, shape, start: int = 0) -> np.ndarray:
    """Host path: elements start .. start+prod(shape)-1 of the stream, as uint16 bits."""
    shape = tuple(int(s) for s in np.atleast_1d(shape)) if not isinstance(shape, int) else (shape,)
    n = int(np.prod(shape)) if shape else 1
    key = np.uint64(stream_key(seed, tensor_id))
    tab = table()
    out = np.empty(n, dtype=np.uint16)
    chunk = 1 << 22
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        i = np.arange(start + c0 + 1, start + c1 + 1, dtype=np.uint64)
        u = _mix64(key + i * np.uint64(GAMMA))
        out[c0:c1] = tab[(u >> np.uint64(64 - TABLE_BITS)).astype(np.int64)]
    return out.reshape(shape)


def rows_bf16(seed: int, tensor_id: int, row_shape, rows) -> np.ndarray:
    """Host path for selected leading-dimension rows of a tensor whose rows hold
    prod(row_shape) elements: returns [len(rows), *row_shape]."""
    row_shape = tuple(row_shape)
    per = int(np.prod(row_shape))
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), per), dtype=np.uint16)
    for j, r in enumerate(rows):
        out[j] = normal_bf16(seed, tensor_id, per, start=int(r) * per)
    return out.reshape((len(rows),) + row_shape)


# ---------------------------------------------------------------------------
# Device path (fills torch tensors on the GPU with the same bits)
# ---------------------------------------------------------------------------
_dev = None
_dev_tables = {}


def build_device() -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = DEV_LIB + ".tmp"
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           DEV_SRC, "-o", tmp], stderr=subprocess.DEVNULL)
    os.replace(tmp, DEV_LIB)
    return DEV_LIB


def _load_dev():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            build_device()
        lib = ctypes.CDLL(DEV_LIB)
        lib.hca_synth_fill_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
        lib.hca_synth_fill_bf16.restype = ctypes.c_int
        _dev = lib
    return _dev


def normal_bf16_device(seed: int, tensor_id: int, shape, device="cuda", start: int = 0):
    """Device path: a torch.bfloat16 tensor holding the same bits as normal_bf16()."""
    import torch
    dev = torch.device(device)
    lib = _load_dev()
    tab = _dev_tables.get(dev)
    if tab is None:
        tab = torch.from_numpy(table().view(np.int16).copy()).to(dev)
        _dev_tables[dev] = tab
    out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    n = out.numel()
    if n:
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.hca_synth_fill_bf16(out.data_ptr(), n, start, stream_key(seed, tensor_id),
                                     tab.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"hca_synth_fill_bf16 failed: {rc}")
    return out
