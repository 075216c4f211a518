"""Host check of the built library's gfx950 code: every DPP instruction reads its DPP
source register at least two wait states after the last vector instruction that wrote
it, the distance the hardware needs and does not enforce by itself (CDNA3/CDNA4 ISA,
"manually inserted wait states": a VALU write of a VGPR followed by a DPP read of it).

The compiler keeps that distance for the DPP operations it emits; the kernels also issue
DPP multiply-adds from inline assembly, which the compiler does not inspect.  This test
disassembles the gfx950 code objects bundled in libsscan.so (code built here) and checks
every DPP instruction, whoever emitted it.  A DPP instruction within two instructions of a
branch target fails the check, since its predecessors are then not known from the listing."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "selective_state_space_sscan_amd", "libsscan.so")
OBJDUMP = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "llvm", "bin", "llvm-objdump")

INSN = re.compile(r"^\s+([a-z_0-9]+)(?:\s+([^/]*?))?\s*//\s*([0-9A-Fa-f]+):")
FUNC = re.compile(r"^([0-9a-f]+) <([^>]+)>:$")
TARGET = re.compile(r"<([^>+]+)\+0x([0-9a-f]+)>")


def _code_objects(tmp):
    lib = os.path.join(tmp, "lib.so")
    shutil.copy(LIB, lib)
    subprocess.run([OBJDUMP, "--offloading", lib], cwd=tmp, check=True, capture_output=True)
    return sorted(os.path.join(tmp, f) for f in os.listdir(tmp) if "amdgcn-amd-amdhsa" in f and "gfx950" in f)


def _regs(tok):
    """VGPR indices named by an operand: v7 or v[4:7]."""
    tok = tok.strip()
    m = re.fullmatch(r"v(\d+)", tok)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def _listing(path):
    out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", path], check=True, capture_output=True, text=True).stdout
    funcs = {}
    insns = []  # (address, mnemonic, operands)
    for line in out.splitlines():
        m = FUNC.match(line)
        if m:
            funcs[m.group(2)] = int(m.group(1), 16)
            continue
        m = INSN.match(line)
        if m:
            insns.append((int(m.group(3), 16), m.group(1), (m.group(2) or ""), line))
    targets = set()
    for _, mn, _, line in insns:
        if mn.startswith("s_cbranch") or mn == "s_branch":
            t = TARGET.search(line)
            if t and t.group(1) in funcs:
                targets.add(funcs[t.group(1)] + int(t.group(2), 16))
    return insns, targets


def _violations(insns, targets):
    bad = []
    checked = 0
    for i, (addr, mn, ops, line) in enumerate(insns):
        if not mn.endswith("_dpp") or not mn.startswith("v_"):
            continue
        checked += 1
        operands = [o for o in ops.split(",")]
        if len(operands) < 2:
            continue
        # the DPP source is the first source operand (VOP1: the only one)
        src = _regs(operands[1].split()[0])
        waits = 0
        j = i
        if addr in targets:
            bad.append(("branch target at a DPP instruction", line))
            continue
        while waits < 2 and j > 0:
            j -= 1
            paddr, pmn, pops, pline = insns[j]
            if pmn == "s_nop":
                waits += int(pops.strip() or "0", 0) + 1
            else:
                if pmn.startswith("v_") and not pmn.startswith(("v_cmp", "v_readlane", "v_readfirstlane")):
                    dst = _regs(pops.split(",")[0].split()[0]) if pops.strip() else set()
                    if dst & src:
                        bad.append((f"{pmn} writes the DPP source {waits} wait state(s) before", line))
                        break
                waits += 1
            if paddr in targets and waits < 2:
                bad.append(("branch target within two instructions before a DPP instruction", line))
                break
    return bad, checked


@pytest.mark.skipif(not os.path.exists(LIB), reason="libsscan.so is not built")
@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="llvm-objdump of ROCm not found")
def test_dpp_sources_are_not_written_within_two_wait_states():
    with tempfile.TemporaryDirectory() as tmp:
        objs = _code_objects(tmp)
        assert objs, "no gfx950 code object in libsscan.so"
        total = 0
        problems = []
        for path in objs:
            insns, targets = _listing(path)
            bad, n = _violations(insns, targets)
            total += n
            problems += bad
        assert total > 1000, f"only {total} DPP instructions found: the listing was not parsed"
        assert not problems, "\n".join(f"{why}: {line.strip()}" for why, line in problems[:20])


def test_checker_flags_a_planted_hazard():
    """The checker itself, on a hand-written listing: a DPP read right after a write of its
    source is flagged, one after an s_nop 1 is not."""
    def ins(addr, text):
        mn, _, ops = text.partition(" ")
        return (addr, mn, ops, f"\t{text} // {addr:012X}: 0")
    hazard = [ins(0, "v_mul_f32_e32 v9, v1, v2"), ins(4, "v_fmac_f32_dpp v10, v9, v15 row_newbcast:0")]
    bad, n = _violations(hazard, set())
    assert n == 1 and len(bad) == 1
    safe = [ins(0, "v_mul_f32_e32 v9, v1, v2"), ins(4, "s_nop 1"), ins(8, "v_fmac_f32_dpp v10, v9, v15 row_newbcast:0")]
    assert _violations(safe, set())[0] == []
    other = [ins(0, "v_mul_f32_e32 v8, v1, v2"), ins(4, "v_fmac_f32_dpp v10, v9, v15 row_newbcast:0")]
    assert _violations(other, set())[0] == []
    ranged = [ins(0, "v_mov_b32_e32 v9, 0"), ins(4, "v_add_f32_e32 v1, v1, v1"),
              ins(8, "v_fmac_f32_dpp v10, v[8:9], v15 row_newbcast:0")]
    assert len(_violations(ranged, set())[0]) == 1
