"""The attention kernel's asynchronous global-to-LDS loads are written in
inline assembly, where the compiler inserts no hazard wait states.  Their
address is an SGPR pair that the compiler fills with v_readfirstlane (a
vector-ALU write of SGPRs), and a vector-memory instruction must not read
such SGPRs within five wait states of that write, or it may use their stale
value as its address.  This test compiles the kernel source to gfx950
assembly (CPU only) and checks every such load."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tree_attention_verification_graft_amd", "csrc", "tree_attention.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


def dma_hazards(asm_text):
    """(loads checked, violations): for each global_load_lds reading
    s[a:b], a vector instruction writing s_a or s_b fewer than five wait
    states before it (s_nop N counts N + 1) is a violation."""
    lines = asm_text.splitlines()
    total, bad = 0, []
    for i, line in enumerate(lines):
        m = re.search(r"global_load_lds_dword(?:x[34])? v\d+, s\[(\d+):(\d+)\]", line)
        if not m:
            continue
        total += 1
        regs = {f"s{k}" for k in range(int(m.group(1)), int(m.group(2)) + 1)}
        ws, j = 0, i - 1
        while j >= 0 and ws < 5:
            t = lines[j].strip()
            j -= 1
            if not t or t.startswith((";", ".")):
                continue
            parts = t.replace(",", " ").split()
            if parts[0] == "s_nop":
                ws += int(parts[1], 0) + 1
                continue
            dst = parts[1] if len(parts) > 1 else ""
            mm = re.match(r"s\[(\d+):(\d+)\]$", dst)
            written = ({f"s{k}" for k in range(int(mm.group(1)), int(mm.group(2)) + 1)}
                       if mm else {dst})
            if parts[0].startswith("v_") and written & regs:
                bad.append((i, ws, t))
                break
            ws += 1
    return total, bad


def test_detector_flags_a_short_distance():
    unsafe = ("v_readfirstlane_b32 s26, v2\n;;#ASMSTART\ns_nop 0\n"
              "global_load_lds_dwordx4 v48, s[26:27]\n")
    safe = ("v_readfirstlane_b32 s26, v2\n;;#ASMSTART\ns_nop 4\n"
            "global_load_lds_dwordx4 v48, s[26:27]\n")
    assert dma_hazards(unsafe)[1] and not dma_hazards(safe)[1]
    # the 4-byte form (the ancestor masks) is checked the same way
    assert dma_hazards(unsafe.replace("dwordx4", "dword"))[1]
    assert dma_hazards(safe.replace("dwordx4", "dword")) == (1, [])


def test_attention_lds_dma_loads_have_their_wait_states(tmp_path):
    flags = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang",
             "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
             "-S", "--cuda-device-only"]
    out = tmp_path / "attn.s"
    r = subprocess.run([HIPCC, *flags, SRC, "-o", str(out)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    total, bad = dma_hazards(out.read_text())
    assert total > 0
    assert not bad, f"{len(bad)} of {total} LDS-DMA loads too close to an SGPR write: {bad[:3]}"
