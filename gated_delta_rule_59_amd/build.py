"""Compile the gfx950 HIP library libgdn2.so in-tree (explicit hipcc line),
and libgdn2_peak.so, the MFMA-rate measurement bench.py reports as context.

All HIP code is built with packed fp32 arithmetic turned off
(-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host pass warns
that it does not know that feature, which is harmless.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn2.so")
SOURCES = ["gdn2_api.hip", "gdn2_fwd.hip", "gdn2_decode.hip", "gdn2_bwd.hip", "gdn2_mixer.hip"]
PEAK_LIB = os.path.join(HERE, "libgdn2_peak.so")
PEAK_SOURCES = ["gdn2_peak.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def hipcc_cmd(out, extra=(), sources=SOURCES):
    return [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *extra, *[os.path.join(CSRC, s) for s in sources], "-o", out]


def _compile(lib, sources, verbose):
    tmp = lib + ".tmp"
    cmd = hipcc_cmd(tmp, sources=sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(x for x in r.stderr.splitlines() if noise not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    _compile(LIB, SOURCES, verbose)
    _compile(PEAK_LIB, PEAK_SOURCES, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
