"""Instruction-level check of the built kernels (CPU: reads the gfx950 code
objects that build() wrote, nothing runs on a GPU).

On gfx9 a vector memory instruction reads its SGPR operands without waiting
for a VALU instruction that writes them (v_readfirstlane and the like); five
wait states must separate the two.  The compiler inserts them before its own
loads, not before the LDS-DMA loads the kernels issue from asm statements, so
every such load whose base a VALU instruction has just formed must carry them
itself.  A base read too early is a stale SGPR: a wild address and a memory
fault.  This test disassembles every kernel object and fails on any vector
memory instruction that reads an SGPR written by a VALU instruction fewer than
five wait states before it."""
import os
import re
import shutil
import subprocess

import pytest

from joint_video_audio_h3_amd import build

LLVM = "/opt/rocm/llvm/bin"
VALU_SGPR_WRITE = re.compile(r"(v_readfirstlane_b32|v_readlane_b32|v_cmp\w*_e64|v_cmpx\w*_e64)\s+s\[?(\d+)(?::(\d+))?")
VMEM = re.compile(r"(global_|buffer_|flat_|scratch_)\w+")
SPAIR = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")


def _sgprs(text):
    out = set()
    for a, b, c in SPAIR.findall(text):
        if c:
            out.add(int(c))
        else:
            out |= set(range(int(a), int(b) + 1))
    return out


def hazards(disasm_lines):
    """(VALU line, VMEM line, wait states) for every violation in a disassembly."""
    ins = []
    for line in disasm_lines:
        t = line.split("//")[0].split(";")[0].strip()
        if t and not t.startswith(".") and not t.endswith(":") and not t.startswith("<"):
            ins.append(t)
    found = []
    for k, t in enumerate(ins):
        m = VALU_SGPR_WRITE.match(t)
        if not m:
            continue
        written = set(range(int(m.group(2)), int(m.group(3) or m.group(2)) + 1))
        waits = 0
        for t2 in ins[k + 1:k + 8]:
            if t2.startswith("s_nop"):
                waits += int(t2.split()[1], 0) + 1
            elif VMEM.match(t2):
                # SGPR operands follow the VGPR address/data operand
                ops = t2.split(None, 1)[1] if " " in t2 else ""
                if written & _sgprs(ops) and waits < 5:
                    found.append((t, t2, waits))
                waits += 1
            else:
                waits += 1
            if waits >= 5:
                break
    return found


def test_scanner_flags_a_planted_case():
    planted = ["v_readfirstlane_b32 s8, v4", "s_add_i32 m0, s10, 0x100", "global_load_lds_dwordx4 v1, s[8:9]"]
    assert len(hazards(planted)) == 1
    guarded = ["v_readfirstlane_b32 s8, v4", "s_nop 4", "global_load_lds_dwordx4 v1, s[8:9]"]
    assert hazards(guarded) == []
    unrelated = ["v_readfirstlane_b32 s7, v4", "global_load_lds_dwordx4 v1, s[8:9]"]
    assert hazards(unrelated) == []


@pytest.mark.timeout(900)
def test_no_valu_sgpr_to_vmem_hazard_in_built_kernels(tmp_path):
    for tool in ("clang-offload-bundler", "llvm-objdump", "llvm-objcopy"):
        if not os.path.exists(os.path.join(LLVM, tool)):
            pytest.skip(f"{tool} not found")
    objs = [os.path.join(build.BUILD, os.path.splitext(s)[0] + ".o") for s in build.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        build.build()
    report = []
    for obj in objs:
        fat = tmp_path / (os.path.basename(obj) + ".fatbin")
        co = tmp_path / (os.path.basename(obj) + ".co")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", obj, os.devnull],
                       check=True, capture_output=True)
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o", f"--input={fat}",
                        f"--targets=hipv4-amdgcn-amd-amdhsa--{build.ARCH}", f"--output={co}"],
                       check=True, capture_output=True)
        dis = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--no-show-raw-insn", str(co)],
                             check=True, capture_output=True, text=True).stdout
        assert "global_load_lds_dwordx4" in dis or "attention" not in obj
        report += [(os.path.basename(obj),) + h for h in hazards(dis.splitlines())]
    assert report == [], "\n".join(map(str, report[:20]))
