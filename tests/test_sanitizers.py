"""Host sanitizer runs (CPU only, no GPU needed).

1. The fp64 oracles (oracle/*.c), built with gcc under AddressSanitizer and
   UndefinedBehaviorSanitizer, run by tests/sanitize/oracle_driver.c: every
   storage dtype, both erase readings, dense and packed batches with empty
   and one-token sequences, and their argument errors.
2. The C ABI's argument validation and workspace sizing (the library's host
   code), built with hipcc with both sanitizers on the host side only, run by
   tests/sanitize/abi_driver.cpp: every entry point's argument errors (all
   return before any launch) and the workspace-size functions over a grid
   that includes INT_MAX-sized arguments.

Any sanitizer report fails the run (-fno-sanitize-recover=all).  The library
build is cached under _build/sanitize, keyed by a hash of its sources.
"""
import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "gated_delta_rule_59_amd", "csrc")
INC = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LIB_SOURCES = ["gdn2_api.hip", "gdn2_fwd.hip", "gdn2_decode.hip", "gdn2_bwd.hip", "gdn2_mixer.hip"]
# sanitizers on the host side of each hipcc line (device code is built as usual)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, timeout, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, **kw)


def test_oracle_under_asan_and_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_san")
    srcs = [os.path.join(ROOT, "oracle", "gdn2_oracle.c"),
            os.path.join(ROOT, "oracle", "gdn2_oracle_bwd.c"),
            os.path.join(SAN, "oracle_driver.c")]
    r = _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-pthread", *srcs,
              "-o", exe, "-lm"], 300)
    assert r.returncode == 0, r.stderr
    r = _run([exe], 300, env=ENV)
    assert r.returncode == 0 and "OK" in r.stdout, r.stdout + r.stderr


def _lib_hash():
    h = hashlib.sha256()
    for f in LIB_SOURCES + ["gdn2_common.hpp", "gdn2_internal.h"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    for f in (os.path.join(INC, "gdn2.h"), os.path.join(SAN, "abi_driver.cpp")):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def test_abi_validation_under_asan_and_ubsan():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    out = os.path.join(ROOT, "_build", "sanitize", _lib_hash())
    exe = os.path.join(out, "abi_san")
    if not os.path.exists(exe):
        os.makedirs(out, exist_ok=True)
        common = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                  "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
                  "-I", INC, "-I", CSRC, "-c"]
        jobs = []
        objs = []
        for f in LIB_SOURCES:
            o = os.path.join(out, f + ".o")
            objs.append(o)
            jobs.append(subprocess.Popen(common + [os.path.join(CSRC, f), "-o", o],
                                         stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
        o = os.path.join(out, "abi_driver.o")
        objs.append(o)
        jobs.append(subprocess.Popen(common + [os.path.join(SAN, "abi_driver.cpp"), "-o", o],
                                     stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
        for j in jobs:
            _, err = j.communicate(timeout=900)
            assert j.returncode == 0, err
        r = _run([HIPCC, "--offload-arch=gfx950", *HOST_SAN[:4], *objs, "-o", exe + ".tmp"], 300)
        assert r.returncode == 0, r.stderr
        os.replace(exe + ".tmp", exe)
    r = _run([exe], 300, env=ENV)
    assert r.returncode == 0 and "OK" in r.stdout, r.stdout + r.stderr
