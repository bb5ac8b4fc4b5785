"""The C ABI's host-side code (validation, row-budget planner, workspace layout, miss
back-off) under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

spec_verify.cpp is rebuilt with the sanitizers on its host code only (each -fsanitize=
follows -Xarch_host; device code is not instrumented), linked with the library's other
objects and with tests/host/sanitize_host_abi.cpp, which drives every host path that
returns before a launch.  No GPU is used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "speculative_decoding_verify_round_amd")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-fno-gpu-sanitize",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def test_host_abi_under_asan_and_ubsan():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    objs = [os.path.join(BUILD, f + ".o") for f in sorted(os.listdir(os.path.join(PKG, "csrc")))
            if f.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library's objects are not built")
    out = os.path.join(BUILD, "sanitize")
    os.makedirs(out, exist_ok=True)
    inc = ["-I" + os.path.join(ROOT, "include")]
    flags = ["-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result", *inc]
    sv = os.path.join(out, "spec_verify_asan.o")
    drv = os.path.join(out, "driver.o")
    exe = os.path.join(out, "sanitize_host_abi")
    for src, obj in ((os.path.join(PKG, "csrc", "spec_verify.cpp"), sv),
                     (os.path.join(ROOT, "tests", "host", "sanitize_host_abi.cpp"), drv)):
        r = subprocess.run([HIPCC, *flags, *SAN, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-fsanitize=address,undefined", "-o", exe, drv, sv, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", LSAN_OPTIONS="suppressions=")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
