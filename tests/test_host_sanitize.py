"""The C ABI layer's host code under AddressSanitizer and UndefinedBehavior-
Sanitizer, on the CPU.

`tests/host/abi_sanitize.cpp` links `csrc/api.hip` (host code instrumented,
`-Xarch_host -fsanitize=...`) with stub kernel launchers that check the launch
descriptors and launch nothing, then calls every entry point with invalid and
(when no GPU is visible) valid arguments.  A sanitizer report aborts the
program; a wrong status fails it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CSRC = os.path.join(ROOT, "block_sparse_spatio_svattn_amd", "csrc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not available")
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"),
              "-I", CSRC, "-Wno-unused-command-line-argument", *SAN]
    objs = []
    for src, extra in [(os.path.join(CSRC, "api.hip"), []),
                       (os.path.join(ROOT, "tests", "host", "abi_sanitize.cpp"), ["-x", "hip"])]:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *common, *extra, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(tmp_path / "abi_sanitize")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN[:4], *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    print(r.stdout)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "OK (0 failures)" in r.stdout
