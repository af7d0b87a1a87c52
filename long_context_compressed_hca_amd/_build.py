"""Build libhca.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libhca.so")
# Measurement support for bench.py --copy-rate (not part of the attention path).
PROBE_LIB = os.path.join(PKG, "libhca_probe.so")
PROBE_SRC = "copy_probe.hip"
SOURCES = ["api.cpp", "compress.hip", "prefill.hip", "decode.hip", "decode_sk.hip", "gate.hip",
           "backward.hip"]
HEADERS = ["hca_common.h", "hca_kernels.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# gfx950 only.  Packed fp32 VALU forms are disabled on purpose.
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _quiet(stderr: str) -> str:
    # hipcc's host pass does not know the gfx950-only feature named above
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False) -> str:
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".", "_") + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.PIPE, text=True)))
    probe_tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", os.path.join(CSRC, PROBE_SRC), "-o", probe_tmp]
    procs.append((PROBE_SRC, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                   stderr=subprocess.PIPE, text=True)))
    failed = []
    for src, cmd, p in procs:
        try:
            out, err = p.communicate(timeout=900)
        except subprocess.TimeoutExpired:
            p.kill()
            out, err = p.communicate()
            failed.append((src, " ".join(cmd), "compiler did not finish within 900 s"))
            continue
        err = _quiet(err)
        if verbose and (out.strip() or err.strip()):
            print(f"[{src}]\n{out}{err}", file=sys.stderr)
        if p.returncode != 0:
            failed.append((src, " ".join(cmd), err))
    if failed:
        msg = "\n\n".join(f"{s}: {c}\n{e}" for s, c, e in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    link = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    if link.returncode != 0:
        raise RuntimeError(f"link failed:\n{_quiet(link.stderr)}")
    os.replace(tmp, LIB)
    os.replace(probe_tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
