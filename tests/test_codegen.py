"""Generated-code checks for the kernels' inline-asm MFMAs (CPU only).

The score MFMAs of the prefill kernel and the two products of its head-mix
epilogue, the decode kernels' products, the backward kernels' chains and the
gate GEMM's MFMAs are inline asm, so the compiler inserts no wait states
around them.  The hardware needs 2 wait states between a VALU write of an
MFMA operand and the MFMA, and some more between the MFMA and a VALU read of
its result.  The kernel sources supply the second (s_nop after the last MFMA
of a chain) and arrange for the first (the operands come from LDS or memory
reads, or the MFMA carries its own s_nop).  These tests compile each kernel
source for gfx950 and check both in the assembly, so a compiler change that
moves a register copy in front of one of these MFMAs is caught on the CPU.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_compressed_hca_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _operands(line):
    return [t.strip() for t in line.split(None, 1)[1].split(",")] if " " in line else []


def _wait_states(line):
    return int(line.split()[1]) + 1 if line.startswith("s_nop") else 1


SOURCES = ["prefill.hip", "decode.hip", "decode_sk.hip", "backward.hip", "gate.hip"]


def _compile(src, tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-S", "--cuda-device-only",
           "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    lines = []
    for raw in out.read_text().splitlines():
        t = raw.split(";")[0].strip()
        if t and not t.startswith(".") and not t.endswith(":"):
            lines.append(t)
    return lines


@pytest.fixture(scope="module")
def prefill_asm(tmp_path_factory):
    return _compile("prefill.hip", tmp_path_factory)


@pytest.fixture(scope="module", params=SOURCES)
def kernel_asm(request, tmp_path_factory):
    return _compile(request.param, tmp_path_factory)


def _vgpr_mfmas(lines):
    for i, l in enumerate(lines):
        if l.startswith("v_mfma") and _operands(l)[0].startswith("v"):
            yield i, l


def test_score_mfmas_present(prefill_asm):
    assert sum(1 for _ in _vgpr_mfmas(prefill_asm)) >= 64


def test_no_valu_write_of_an_operand_just_before_an_asm_mfma(prefill_asm):
    bad = []
    for i, l in _vgpr_mfmas(prefill_asm):
        srcs = set().union(*[_regs(t) for t in _operands(l)[1:4]])
        ws = 0
        for j in range(i - 1, max(0, i - 8), -1):
            p = prefill_asm[j]
            if ws >= 2:
                break
            if p.startswith("v_") and not p.startswith("v_mfma"):
                ops = _operands(p)
                if ops and _regs(ops[0]) & srcs:
                    bad.append((p, l))
            ws += _wait_states(p)
    assert not bad, bad[:5]


def test_no_valu_write_of_any_operand_just_before_an_mfma(kernel_asm):
    # every MFMA, also those accumulating into AGPRs (the head-mix product of the
    # prefill epilogue, the decode and backward products are inline asm of that
    # kind): no VALU write, v_accvgpr_write included, of a source operand
    # within 2 wait states
    prefill_asm = kernel_asm
    bad = []
    for i, l in enumerate(prefill_asm):
        if not l.startswith("v_mfma"):
            continue
        srcs = set().union(*[_regs(t) for t in _operands(l)[1:4]])
        ws = 0
        for j in range(i - 1, max(0, i - 8), -1):
            p = prefill_asm[j]
            if ws >= 2:
                break
            if p.startswith("v_") and not p.startswith("v_mfma"):
                ops = _operands(p)
                if ops and _regs(ops[0]) & srcs:
                    bad.append((p, l))
            ws += _wait_states(p)
    assert not bad, bad[:5]


def test_chain_results_wait_before_valu_reads(kernel_asm):
    # after an MFMA writing VGPRs, the first instruction that reads them must be
    # at least 18 wait states later (another MFMA of the same chain excepted)
    prefill_asm = kernel_asm
    bad = []
    for i, l in _vgpr_mfmas(prefill_asm):
        dst = _regs(_operands(l)[0])
        ws = 0
        for j in range(i + 1, min(len(prefill_asm), i + 40)):
            p = prefill_asm[j]
            if p.startswith("v_mfma") and _operands(p)[0] == _operands(l)[0]:
                break  # next MFMA of the chain (accumulates in place)
            ops = _operands(p)
            if ops and not p.startswith("s_") and (set().union(*[_regs(t) for t in ops[1:]]) & dst
                                                    or (p.startswith("v_") and _regs(ops[0]) & dst)):
                if ws < 18:
                    bad.append((l, p, ws))
                break
            ws += _wait_states(p)
            if ws >= 18:
                break
    assert not bad, bad[:5]
