"""Wait states around the inline-assembly matrix instructions (CPU: compile and scan).

The dK/dV and dQ kernels issue some v_mfma_f32_32x32x16_bf16 as inline assembly with their
accumulators in AGPRs (common.hpp, mfma32_agpr2), with no wait states ahead of them.  The
compiler does not model hazards for inline assembly, so this test compiles those sources to
gfx950 assembly with the library's own flags and checks, over the whole instruction stream:

- no vector-ALU instruction writes a source register (A, B or C) of a matrix instruction
  within the two instructions before it (the hardware needs two wait states there);
- no matrix instruction's result feeds another's A or B operand within 20 instructions
  (such a read must wait for the first one to retire);
- no inline-assembly matrix instruction follows a label within two wait states, where the
  tail of a predecessor block could supply the write (the compiler's own matrix instructions
  get their wait states across block edges from the compiler);
- nothing but another matrix instruction accumulating into exactly the same registers reads
  or writes an inline-assembly matrix instruction's result within RESULT_WAIT wait states
  after it (the compiler, which does not know the instruction is still running, may copy or
  spill an accumulator that it believes is ready: that reads a stale value).
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from suffix_attention_amd import build

SOURCES = ["attn_mfma_bwd.hip", "attn_mfma_dq.hip", "attn_mfma_dqs.hip", "attn_mfma_fwd.hip", "attn_mfma_fwd_dq.hip"]
# wait states from a 16-pass matrix instruction to a vector read or write of its result
RESULT_WAIT = 18


def _regs(tok: str) -> set:
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _operands(inst: str) -> list:
    parts = inst.split(None, 1)
    return [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []


def _stream(asm: str) -> tuple:
    """Instructions in text order (a label is kept as the marker ':'), and the set of indices
    of those that come from inline assembly."""
    out, inline, in_asm = [], set(), False
    for line in asm.split("\n"):
        if ";;#ASMSTART" in line:
            in_asm = True
        elif ";;#ASMEND" in line:
            in_asm = False
        s = line.split(";")[0].strip()
        if not s or (s.startswith(".") and not s.endswith(":")):
            continue
        if in_asm:
            inline.add(len(out))
        out.append(":" if s.endswith(":") else s)
    return out, inline


def _scan(insts: list, inline=None) -> list:
    """inline: indices of the inline-assembly instructions (None: treat all as inline)."""
    problems = []
    for i, s in enumerate(insts):
        if not s.startswith("v_mfma"):
            continue
        is_inline = inline is None or i in inline
        ops = _operands(s)
        srcs = set().union(*(_regs(o) for o in ops[1:4]))
        ab = _regs(ops[1]) | _regs(ops[2])
        # walk back until two wait states separate the instruction from anything earlier:
        # each instruction is at least one, s_nop k is k + 1
        states, j = 0, 1
        while states < 2 and i - j >= 0:
            p = insts[i - j]
            if p == ":":
                if is_inline:
                    problems.append(f"matrix instruction right after a label: {s}")
                break
            if p.startswith("v_") and not p.startswith("v_mfma") and _regs(_operands(p)[0]) & srcs:
                problems.append(f"VALU write then matrix read: {p} => {s}")
            m = re.match(r"s_nop\s+(\d+)", p)
            states += int(m.group(1)) + 1 if m else 1
            j += 1
        for j in range(1, min(20, i) + 1):
            p = insts[i - j]
            if p.startswith("v_mfma") and _regs(_operands(p)[0]) & ab:
                problems.append(f"matrix result feeds a matrix operand: {p} => {s}")
        if is_inline:
            dst = _regs(ops[0])
            states, j = 0, 1
            while states < RESULT_WAIT and i + j < len(insts):
                p = insts[i + j]
                j += 1
                if p == ":":
                    continue
                m = re.match(r"s_nop\s+(\d+)", p)
                states += int(m.group(1)) + 1 if m else 1
                if p.startswith("s_"):
                    continue
                pops = _operands(p)
                touched = set().union(set(), *(_regs(o) for o in pops))
                if not touched & dst:
                    continue
                if p.startswith("v_mfma") and _regs(pops[0]) == dst and _regs(pops[3]) == dst \
                        and not (_regs(pops[1]) | _regs(pops[2])) & dst:
                    continue  # back-to-back accumulation into the same registers
                problems.append(f"matrix result touched while in flight: {s} => {p}")
    return problems


def test_scanner_catches_planted_hazards():
    # the scanner itself: a VALU write of an operand one instruction ahead must be reported,
    # one three instructions ahead must not
    bad = ["v_cvt_pk_bf16_f32 v4, v1, v2", "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"]
    ok = ["v_cvt_pk_bf16_f32 v4, v1, v2", "s_add_u32 s0, s0, 1", "ds_read_b128 v[20:23], v30",
          "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"]
    chain = ["v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
             "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[8:11], a[0:15]"]
    assert _scan(bad)
    assert not _scan(ok)
    assert _scan(chain)
    # one wait state is not enough, two are
    assert _scan([bad[0], "s_nop 0", bad[1]])
    assert not _scan([bad[0], "s_nop 1", bad[1]])
    # a label right ahead counts against inline assembly only
    after_label = ["s_add_u32 s0, s0, 1", ":", bad[1]]
    assert _scan(after_label, inline={2})
    assert not _scan(after_label, inline=set())
    src = "\n".join(["s_add_u32 s0, s0, 1", ".LBB0_1:", ";;#ASMSTART", bad[1], ";;#ASMEND"])
    assert _scan(*_stream(src))
    # an accumulator copied out (or overwritten) right after an inline matrix instruction
    # writes it is caught; the same copy after enough wait states, or a chained accumulation,
    # is not
    mm = "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"
    assert _scan([mm, "s_nop 0", "v_accvgpr_read_b32 v20, a3"], inline={0})
    assert _scan([mm, "v_accvgpr_mov_b32 a15, a31"], inline={0})
    assert _scan([mm, "scratch_store_dwordx4 off, a[0:3], off"], inline={0})
    assert not _scan([mm, "s_nop 7", "s_nop 7", "s_nop 1", "v_accvgpr_read_b32 v20, a3"], inline={0})
    assert not _scan([mm, mm, "v_accvgpr_read_b32 v20, a16"], inline={0, 1})


@pytest.mark.skipif(shutil.which(build.HIPCC) is None and not os.path.exists(build.HIPCC),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_inline_matrix_instructions_have_their_wait_states(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [build.HIPCC, *build.FLAGS, *build.PER_SOURCE.get(src, []), "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    insts, inline = _stream(out.read_text())
    n_mfma = sum(1 for s in insts if s.startswith("v_mfma"))
    assert n_mfma > 100, "expected the matrix kernels in the assembly"
    assert any(insts[i].startswith("v_mfma") for i in inline), "expected inline matrix instructions"
    problems = _scan(insts, inline)
    assert not problems, "\n".join(problems[:20])
