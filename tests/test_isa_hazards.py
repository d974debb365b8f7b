"""The gfx950 scaled MFMA reads its operand registers (notably the per-lane
E8M0 scale registers) for several cycles after issue, and the compiler does
not keep those registers untouched afterwards.  The expert GEMMs therefore
issue it from inline assembly followed by 32 wait states.  This test builds
the GEMM source for gfx950 and checks, in the generated AMD assembly, that no
instruction writes an operand register of a scaled MFMA within 32 wait
states of it.  CPU-only: hipcc cross-compiles."""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "block_scaled_fp4_sqrtsoftplus_amd", "csrc", "expert_gemm.hip")
HIPCC = "/opt/rocm/bin/hipcc"
NEED = 32


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


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_scaled_mfma_operands_untouched_for_32_wait_states():
    tmp = tempfile.mkdtemp()
    try:
        cmd = [HIPCC, "--offload-arch=gfx950", "--cuda-device-only", "-S", "-O3", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=off",
               "-I", os.path.join(ROOT, "include"), "-I", os.path.dirname(SRC), SRC,
               "-o", os.path.join(tmp, "eg.s")]
        subprocess.run(cmd, check=True, capture_output=True)
        asm = open(os.path.join(tmp, "eg.s")).read()
    finally:
        shutil.rmtree(tmp)
    funcs = _functions(asm)
    total = 0
    for name, ins in funcs.items():
        for i, s in enumerate(ins):
            if not s.startswith("v_mfma_scale"):
                continue
            total += 1
            ops = [o.strip() for o in s.split(None, 1)[1].split(" op_sel")[0].split(",")]
            watch = _regs(ops[1]) | _regs(ops[2]) | _regs(ops[4]) | _regs(ops[5])
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
                    dst = parts[1].split(",")[0].strip()
                    assert not (_regs(dst) & watch), f"{name}: '{t}' {ws} wait states after '{s}'"
    assert total > 0
