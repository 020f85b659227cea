"""The direct HBM->LDS loads are inline assembly, which the compiler does not
pad for hazards.  A vector-memory instruction may read an SGPR only 5 wait
states after a VALU instruction wrote it (the tile base address often comes
from v_readfirstlane), and the LDS-direct load reads M0 one wait state after
it is written.  The kernels' asm block therefore starts with s_nop 4; a build
without it read a stale base address and faulted the GPU.  This test
disassembles the gfx950 code objects of this repository's own build and
checks every global_load_lds instruction: an s_nop of at least 4 right
before it, and, walking back through straight-line code, at least 5 wait
states since the last VALU write of its base SGPRs and at least 1 since the
last write of M0.  CPU only."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "long_context_sequence_dfa_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

INSN = re.compile(r"^\s+([a-z_0-9]+)(?:\s+([^/]*?))?\s*//")
LABEL = re.compile(r"^\S.*:\s*$|^<.*>:")


def sgprs(operand):
    """SGPR numbers named by an operand (s7, s[4:5]); empty for others."""
    m = re.fullmatch(r"s(\d+)", operand)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def parse(lines):
    """(mnemonic, operand list) per instruction line; None marks a label."""
    out = []
    for ln in lines:
        if LABEL.match(ln):
            out.append(None)
            continue
        m = INSN.match(ln)
        if m:
            ops = [o.strip() for o in (m.group(2) or "").split(",") if o.strip()]
            out.append((m.group(1), ops))
    return out


def wait_states(mn, ops):
    if mn == "s_nop":
        return int(ops[0], 0) + 1 if ops else 1
    return 1


def check(insns):
    """Problems found in a parsed instruction list (empty: none)."""
    problems = []
    for i, ins in enumerate(insns):
        if ins is None or not ins[0].startswith("global_load_lds"):
            continue
        mn, ops = ins
        base = sgprs(ops[1]) if len(ops) > 1 else set()
        prev = insns[i - 1] if i > 0 else None
        if prev is None or prev[0] != "s_nop" or wait_states(*prev) < 5:
            problems.append((i, mn, "not preceded by s_nop >= 4"))
        ws, j = 0, i - 1
        while j >= 0 and insns[j] is not None and ws < 5:
            pm, pops = insns[j]
            dst = pops[0] if pops else ""
            if pm.startswith("v_") and sgprs(dst) & base and ws < 5:
                problems.append((i, mn, f"VALU write of its base {dst} {ws} wait states before"))
            if dst == "m0" and ws < 1:
                problems.append((i, mn, "M0 written right before"))
            ws += wait_states(pm, pops)
            j -= 1
    return problems


def disassemble(obj, tmp_path):
    fat = tmp_path / (os.path.basename(obj) + ".fatbin")
    co = tmp_path / (os.path.basename(obj) + ".co")
    subprocess.check_call([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fat}", obj])
    subprocess.check_call([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o",
                           f"--input={fat}", f"--targets={TARGET}", f"--output={co}"])
    return subprocess.check_output([f"{LLVM}/llvm-objdump", "-d", "--mcpu=gfx950", str(co)],
                                   text=True).splitlines()


def objects():
    if not os.path.isdir(BUILD) or not any(f.endswith(".hip.o") for f in os.listdir(BUILD)):
        from long_context_sequence_dfa_amd import _build
        _build.build()
    return sorted(os.path.join(BUILD, f) for f in os.listdir(BUILD) if f.endswith(".hip.o"))


@pytest.mark.skipif(not os.path.exists(f"{LLVM}/llvm-objdump"), reason="no ROCm LLVM tools")
def test_every_direct_lds_load_is_padded(tmp_path):
    total = 0
    for obj in objects():
        insns = parse(disassemble(obj, tmp_path))
        n = sum(1 for x in insns if x is not None and x[0].startswith("global_load_lds"))
        total += n
        assert check(insns) == [], os.path.basename(obj)
    # the forward, dQ and dK/dV kernels all stream tiles this way
    assert total > 1000


def test_the_scan_catches_a_missing_pad():
    good = """
\tv_readfirstlane_b32 s46, v2                 // 0000: 7E5C0502
\ts_mov_b32 m0, s84                           // 0004: BEFC0054
\ts_nop 4                                     // 0008: BF800004
\tglobal_load_lds_dwordx4 v6, s[46:47]        // 000C: DDF48000 002E0006
""".splitlines()
    assert check(parse(good)) == []
    no_nop = [ln for ln in good if "s_nop" not in ln]
    probs = check(parse(no_nop))
    assert any("s_nop" in p[2] for p in probs)
    assert any("VALU write" in p[2] for p in probs)
    assert any("M0" in p[2] for p in probs)
    short = [ln.replace("s_nop 4", "s_nop 2") for ln in good]
    assert any("VALU write" in p[2] for p in check(parse(short)))
