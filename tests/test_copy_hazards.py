"""The direct global -> LDS copies are issued from inline assembly, whose
operands the compiler's hazard checks do not see.  Every copy in the
generated gfx950 code must sit at least 5 wait states after a vector
instruction that wrote a scalar register of its address, and at least 1
after a scalar write of M0 (its LDS destination).  With fewer, the copy can
read a stale base address: a base formed in vector registers and moved to
scalar ones right before the copy is how the history-layout attention
instances once faulted the device.  (No GPU: the kernels are compiled to
assembly and read.)"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dilated_sparse_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def copy_hazards(asm_lines):
    lines = [x.strip() for x in asm_lines if x.strip() and not x.strip().startswith((";", "."))]
    copies, bad = 0, []
    for i, line in enumerate(lines):
        if not line.startswith("global_load_lds"):
            continue
        copies += 1
        m = re.search(r"s\[(\d+):(\d+)\]", line)
        base = {f"s{m.group(1)}", f"s{m.group(2)}"} if m else set()
        waits = 0
        for k in range(1, 8):
            prev = lines[i - k]
            if prev.startswith("s_nop"):
                waits += int(prev.split()[1]) + 1
                continue
            toks = prev.replace(",", " ").split()
            dst = toks[1] if len(toks) > 1 else ""
            if prev.startswith("v_") and dst in base and waits < 5:
                bad.append(lines[i - k:i + 1])
                break
            if prev.startswith("s_") and dst == "m0" and waits < 1:
                bad.append(lines[i - k:i + 1])
                break
            waits += 1
    return copies, bad


@pytest.mark.parametrize("src", ["attn_prefill.hip", "scan.hip"])
def test_copies_have_their_wait_states(src, tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not available")
    out = tmp_path / "k.s"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-S", "--cuda-device-only",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
                    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, os.path.join(CSRC, src), "-o", str(out)],
                   check=True, capture_output=True)
    copies, bad = copy_hazards(out.read_text().splitlines())
    assert copies > 0
    assert not bad, bad[:3]


def test_scan_flags_a_missing_wait():
    """The check itself: a base written by v_readfirstlane right before the
    copy, and M0 written right before it, are both reported."""
    asm = ["v_readfirstlane_b32 s23, v7", "global_load_lds_dwordx4 v3, s[22:23]",
           "s_mov_b32 m0, s4", "global_load_lds_dwordx4 v3, off",
           "v_readfirstlane_b32 s9, v1", "s_mov_b32 m0, s2", "s_nop 4", "global_load_lds_dwordx4 v2, s[8:9]"]
    copies, bad = copy_hazards(asm)
    assert copies == 3 and len(bad) == 2
