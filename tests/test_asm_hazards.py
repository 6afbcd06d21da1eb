"""Device-assembly check of the HIP sources (host only: hipcc cross-compiles).

The kernels use inline assembly (DPP multiply scans, register retirement).
The compiler inserts the wait states a transcendental's result needs
(v_rcp, v_exp, ...) before its own readers, but not before an inline-assembly
block, and a block that read a v_rcp_f32 result two to four instructions later
was measured to see stale values.  This test compiles the library sources to
gfx950 assembly and checks that no inline-assembly block reads a
transcendental's result within the next 11 instructions.
"""
import os
import re
import shutil
import subprocess

import pytest

from gated_delta_rule_59_amd import build

TRANS = ("v_rcp_", "v_exp_", "v_log_", "v_sqrt_", "v_rsq_", "v_sin_", "v_cos_")
WINDOW = 11


def _vregs(text):
    regs = set()
    for a, b in re.findall(r"v\[(\d+):(\d+)\]", text):
        regs |= set(range(int(a), int(b) + 1))
    for a in re.findall(r"\bv(\d+)\b", text):
        regs.add(int(a))
    return regs


def _instructions(asm_text):
    """(text, inside inline assembly) for each instruction, in order."""
    out, inside = [], False
    for line in asm_text.split("\n"):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            inside = True
            continue
        if t.startswith(";;#ASMEND"):
            inside = False
            continue
        if not line.startswith("\t") or not t or t.startswith((";", ".")):
            continue
        out.append((t, inside))
    return out


def trans_reads_by_inline_asm(asm_text, window=WINDOW):
    ins = _instructions(asm_text)
    bad = []
    for i, (t, _) in enumerate(ins):
        if not t.startswith(TRANS):
            continue
        parts = t.split(None, 1)
        dst = _vregs(parts[1].split(",")[0]) if len(parts) > 1 else set()
        for d in range(1, window + 1):
            if i + d >= len(ins):
                break
            t2, in_asm = ins[i + d]
            p2 = t2.split(None, 1)
            if in_asm and len(p2) > 1 and dst & _vregs(p2[1]):
                bad.append((t, d, t2))
    return bad


def test_checker_finds_a_planted_case():
    planted = "\n".join([
        "\tv_rcp_f32_e32 v7, v3",
        "\tv_mul_f32_e32 v1, v2, v2",
        ";;#ASMSTART",
        "\tv_fma_mixhi_f16 v9, v4, v7, 0",
        ";;#ASMEND",
        "\tv_rcp_f32_e32 v8, v3",
        "\tv_mul_f32_e32 v5, v8, v2",
    ])
    bad = trans_reads_by_inline_asm(planted)
    assert len(bad) == 1 and bad[0][1] == 2


@pytest.mark.parametrize("src", ["gdn2_fwd.hip", "gdn2_decode.hip"])
def test_no_transcendental_result_feeds_inline_asm(src, tmp_path):
    if not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    cmd = [build.HIPCC, f"--offload-arch={build.ARCH}", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(build.ROOT, "include"), "-I", build.CSRC,
           "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    bad = trans_reads_by_inline_asm(out.read_text())
    assert not bad, bad[:5]
