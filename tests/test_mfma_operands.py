"""The attention kernel's MFMAs never write a register that is also one of
their A/B sources.

A 32x32 MFMA reads its sources over several passes while it writes its
result, so a destination that overlaps a source gives wrong results; the
kernel keeps each operand alive past its last MFMA (an empty asm statement)
so that the register allocator cannot do that. This test compiles the
kernel to gfx950 assembly with the same flags as the library and checks
every v_mfma instruction. CPU only (hipcc cross-compiles).
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_mixed_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_attention_mfma_destinations_never_overlap_sources(tmp_path):
    out = tmp_path / "attn.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, "attn.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    n, bad = 0, []
    for line in out.read_text().splitlines():
        s = line.strip()
        if not s.startswith("v_mfma"):
            continue
        n += 1
        ops = [t.strip() for t in s.split(None, 1)[1].split(",")]
        d, a, b = _regs(ops[0]), _regs(ops[1]), _regs(ops[2])
        if d & (a | b):
            bad.append(s)
    assert n >= 100, f"only {n} MFMA instructions found"
    assert not bad, "\n".join(bad[:10])
