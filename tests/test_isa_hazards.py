"""The expert GEMMs issue the gfx950 scaled MFMA from inline assembly and
close each group of MFMAs with 32 wait states, so that no later instruction
overwrites a register the MFMA may still read: the compiler does not see the
MFMA inside the asm and would not hold such writes back.  (A streaming GEMM
that let the compiler reuse a per-lane E8M0 scale register right after the
MFMA produced wrong rows; overwriting the A or B data registers with the
next VALU instruction has been measured harmless on gfx950.)  This test
builds the GEMM source for gfx950 and checks, in the generated AMD assembly,
that no VALU instruction writes a scale register or the accumulator of a
scaled MFMA within 32 wait states of it, and that nothing but another MFMA
reads an MFMA's accumulator within that distance.  Before the MFMA, the
hardware needs wait states between a VALU write of a source register (A, B,
the accumulator or a scale) and the MFMA's read of it -- the compiler puts
two there for the builtin -- which it cannot insert in front of an asm MFMA
either: the check asks for at least PRE wait states there.  (A W4AFP8 GEMM whose B operand was
written by the VALU instruction right before the asm MFMA read a stale value
on gfx950.)  CPU-only: hipcc cross-compiles."""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_fp4_sqrtsoftplus_amd", "csrc")
SOURCES = ["expert_gemm.hip", "expert_gemm_w4.hip"]
HIPCC = "/opt/rocm/bin/hipcc"
NEED = 32
PRE = 2


def _regs(op):
    m = re.match(r"([va])\[(\d+):(\d+)\]", op)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {op} if re.match(r"[va]\d+$", op) else set()


def _functions(asm):
    funcs, cur = {}, None
    for line in asm.split("\n"):
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur = m.group(1)
            funcs[cur] = []
        elif cur and line.startswith("\t") and not line.startswith("\t.") and not line.strip().startswith(";"):
            funcs[cur].append(line.strip())
    return funcs


def _compile(src):
    tmp = tempfile.mkdtemp()
    try:
        cmd = [HIPCC, "--offload-arch=gfx950", "--cuda-device-only", "-S", "-O3", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=off",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, src),
               "-o", os.path.join(tmp, "eg.s")]
        subprocess.run(cmd, check=True, capture_output=True)
        return open(os.path.join(tmp, "eg.s")).read()
    finally:
        shutil.rmtree(tmp)


def _written(t):
    """Registers a VALU instruction writes (none for other instructions)."""
    if not t.startswith("v_") or t.startswith("v_mfma"):
        return set()
    parts = t.split(None, 1)
    return _regs(parts[1].split(",")[0].strip()) if len(parts) == 2 else set()


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", SOURCES)
def test_scaled_mfma_sources_settled_before_issue(src):
    funcs = _functions(_compile(src))
    total = 0
    for name, ins in funcs.items():
        for i, s in enumerate(ins):
            if not s.startswith("v_mfma_scale"):
                continue
            total += 1
            ops = [o.strip() for o in s.split(None, 1)[1].split(" op_sel")[0].split(",")]
            srcs = _regs(ops[1]) | _regs(ops[2]) | _regs(ops[3]) | _regs(ops[4]) | _regs(ops[5])
            ws = 0
            for t in reversed(ins[:i]):
                if ws >= PRE:
                    break
                assert not (_written(t) & srcs), f"{name}: '{t}' {ws} wait states before '{s}'"
                m = re.match(r"s_nop (\d+)", t)
                ws += int(m.group(1)) + 1 if m else 1
    assert total > 0


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", SOURCES)
def test_scaled_mfma_operands_untouched_for_32_wait_states(src):
    funcs = _functions(_compile(src))
    total = 0
    for name, ins in funcs.items():
        for i, s in enumerate(ins):
            if not s.startswith("v_mfma_scale"):
                continue
            total += 1
            ops = [o.strip() for o in s.split(None, 1)[1].split(" op_sel")[0].split(",")]
            watch = _regs(ops[0]) | _regs(ops[4]) | _regs(ops[5])
            ws = 0
            for t in ins[i + 1:]:
                if ws >= NEED:
                    break
                m = re.match(r"s_nop (\d+)", t)
                if m:
                    ws += int(m.group(1)) + 1
                    continue
                ws += 1
                if t.startswith(("global_load", "buffer_load", "ds_read", "s_", "global_store", "ds_write")):
                    continue
                parts = t.split(None, 1)
                if len(parts) == 2:
                    args = [a.strip() for a in parts[1].split(",")]
                    assert not (_regs(args[0]) & watch), f"{name}: '{t}' {ws} wait states after '{s}'"
                    if not t.startswith("v_mfma"):
                        # no read of the accumulator before the result is final
                        read = set().union(*(_regs(a.split()[0]) for a in args[1:] if a))
                        assert not (read & _regs(ops[0])), f"{name}: '{t}' reads the result {ws} wait states after '{s}'"
    assert total > 0
