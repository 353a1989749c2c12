"""The generated gfx950 assembly of every kernel source has no inline-asm
VALU instruction that reads a VGPR whose last writer is a matrix-core (MFMA)
instruction.

The compiler inserts the wait states an MFMA result needs before a dependent
VALU read only for instructions it generates; an inline-asm reader gets none
and can see stale register contents.  The scan walks each function in
program order (straight line, which over-approximates across branches) and
tracks the last writer of every VGPR.  Runs on the CPU: hipcc cross-compiles.
"""
import os
import re
import shutil
import subprocess

import pytest

from visual_kv_pruning_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")

_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
_WRITES = ("v_", "ds_read", "buffer_load", "global_load", "flat_load", "scratch_load")


def _regs(tok):
    out = []
    for m in _VREG.finditer(tok):
        if m.group(3) is not None:
            out.append(int(m.group(3)))
        else:
            out.extend(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def scan(asm_text):
    """Returns [(function, instruction)] for inline-asm VALU reads of MFMA results."""
    found = []
    func, last, in_asm = "?", {}, False
    for line in asm_text.split("\n"):
        if re.match(r"^[A-Za-z_][\w.$]*:\s*(;.*)?$", line) and not line.startswith("."):
            func, last = line.split(":")[0], {}
            continue
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith((";", ".")):
            continue
        parts = t.split(None, 1)
        op = parts[0]
        ops = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
        if not ops:
            continue
        dst, srcs = _regs(ops[0]), [r for o in ops[1:] for r in _regs(o)]
        if in_asm and op.startswith("v_") and any(last.get(r) == "mfma" for r in srcs):
            found.append((func, t))
        if op.startswith(_WRITES):
            kind = "mfma" if op.startswith("v_mfma") else "other"
            for r in dst:
                last[r] = kind
    return found


def test_scanner_flags_a_planted_hazard():
    asm = "\n".join([
        "kern:",
        "\tv_mfma_f32_16x16x32_bf16 v[8:11], v[0:3], v[4:7], 0",
        "\t;;#ASMSTART",
        "\tv_max_f32 v12, v8, v9",
        "\t;;#ASMEND",
        "\tv_add_f32_e32 v13, v10, v11",
    ])
    assert scan(asm) == [("kern", "v_max_f32 v12, v8, v9")]
    # a compiler-generated read in between makes the asm read safe
    safe = asm.replace("\t;;#ASMSTART", "\tv_mov_b32_e32 v8, v8\n\tv_mov_b32_e32 v9, v9\n\t;;#ASMSTART")
    assert scan(safe) == []


@pytest.mark.parametrize("src", [os.path.basename(s) for s in build.sources()])
def test_no_inline_asm_reads_of_mfma_results(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [build.HIPCC, *build.FLAGS, *build.EXTRA.get(src, []), "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    found = scan(out.read_text())
    assert not found, f"{src}: inline asm reads MFMA results: {found[:5]}"
