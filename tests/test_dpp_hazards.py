"""The reverse pass issues some of its broadcast FMAs (v_fmac_f32_dpp, inline
asm) without their own s_nop: a DPP read of a VGPR needs two wait states
after the VALU op that wrote it, and the compiler does not see into the asm.
This compiles the backward's kernels to gfx950 assembly (no GPU needed) and
checks every v_fmac_f32_dpp: its broadcast source must not have been written
by a VALU op within the two preceding wait states."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_scan_amd", "csrc")


def _regs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def dpp_fmac_hazards(lines):
    """(number of v_fmac_f32_dpp checked, list of hazards, label crossings)."""
    hazards, crossings, checked = [], [], 0
    for i, line in enumerate(lines):
        t = line.strip()
        if not t.startswith("v_fmac_f32_dpp"):
            continue
        checked += 1
        src = _regs(t.split(None, 1)[1].split(",")[1])
        waits, j = 0, i - 1
        while waits < 2 and j >= 0:
            u = lines[j].strip()
            j -= 1
            if not u or u.startswith(";"):
                continue
            if u.startswith(".") and u.endswith(":") or re.match(r"^\.LBB\w+:", u):
                crossings.append((i, t))
                break
            if u.startswith("."):
                continue
            mnem = u.split()[0]
            if mnem == "s_nop":
                waits += int(u.split()[1]) + 1
                continue
            if mnem.startswith("v_"):
                ops = u.split(None, 1)[1].split(",")
                written = _regs(ops[0])
                if "swap" in mnem:
                    written |= _regs(ops[1])
                if written & src:
                    hazards.append((i, t, u))
            waits += 1
    return checked, hazards, crossings


def test_checker_finds_a_planted_hazard():
    lines = ["v_mul_f32_e32 v5, v1, v2",
             "v_fmac_f32_dpp v7, v5, v3 row_newbcast:3 row_mask:0xf bank_mask:0xf"]
    assert len(dpp_fmac_hazards(lines)[1]) == 1
    lines.insert(1, "s_nop 1")
    assert dpp_fmac_hazards(lines)[1] == []


def test_reverse_pass_broadcast_fmacs_have_their_wait_states(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / "ss_bwd.s"
    cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip", "--cuda-device-only",
           "-S", os.path.join(CSRC, "ss_bwd.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    checked, hazards, crossings = dpp_fmac_hazards(out.read_text().split("\n"))
    assert checked > 1000
    assert hazards == [], hazards[:5]
    assert crossings == [], crossings[:5]
