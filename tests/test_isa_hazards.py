"""The bf16 forward keeps the P V accumulators in AGPRs through an inline-asm
MFMA, which the compiler cannot see into.  This test compiles the kernel to
gfx950 assembly and checks that no instruction other than the same
accumulator's next MFMA touches an accumulator within the MFMA's result
latency (counted conservatively as 19 wait states), so that no register
allocation choice (copy, spill, rescale) reads or overwrites it early.
Runs on the CPU (hipcc cross-compiles)."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "exact_attention_101_amd", "csrc", "fa_fwd_bf16.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LATENCY = 19


def _agprs(text):
    regs = set()
    for a, b in re.findall(r"a\[(\d+):(\d+)\]", text):
        regs |= set(range(int(a), int(b) + 1))
    for a in re.findall(r"\ba(\d+)\b", text):
        regs.add(int(a))
    return regs


def _hazards(asm_lines):
    found = []
    for i, line in enumerate(asm_lines):
        m = re.match(r"\s+v_mfma\w* a\[(\d+):(\d+)\],", line)
        if not m:
            continue
        dst = set(range(int(m.group(1)), int(m.group(2)) + 1))
        ws, j = 0, i + 1
        while j < len(asm_lines) and ws < LATENCY:
            t = asm_lines[j].strip()
            j += 1
            if not t or t.startswith((";", ".")):
                continue
            if t.startswith("s_nop"):
                ws += int(t.split()[1]) + 1
                continue
            ws += 1
            if t.startswith("s_"):
                continue
            if t.startswith("v_mfma"):
                mm = re.match(r"v_mfma\w* a\[(\d+):(\d+)\],.*, a\[(\d+):(\d+)\]$", t)
                if mm:
                    d2 = set(range(int(mm.group(1)), int(mm.group(2)) + 1))
                    c2 = set(range(int(mm.group(3)), int(mm.group(4)) + 1))
                    if (d2 & dst and d2 != dst) or (c2 & dst and c2 != dst):
                        found.append((line.strip(), t))
                continue
            if _agprs(t) & dst:
                found.append((line.strip(), t))
    return found


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_no_early_accumulator_access(tmp_path):
    import exact_attention_101_amd.build as build
    out = tmp_path / "fa_fwd_bf16.s"
    cmd = [HIPCC, *build.FLAGS_DEVICE_ASM, "-o", str(out), SRC]
    subprocess.run(cmd, check=True, capture_output=True, cwd=tmp_path)
    lines = out.read_text().split("\n")
    mfmas = [l for l in lines if re.match(r"\s+v_mfma\w* a\[", l)]
    assert mfmas, "no AGPR-accumulator MFMA found"
    found = _hazards(lines)
    assert not found, found[:5]
