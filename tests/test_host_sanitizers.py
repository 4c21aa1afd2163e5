"""The host code of the bit-allocation search under sanitizers (CPU only).

ddg_pd_allocate runs its restarts on host threads.  tests/host/pd_search_driver.cpp
calls it at several targets; it is built with hipcc from the library's own
pd.hip, with the host code instrumented (ThreadSanitizer; AddressSanitizer with
UndefinedBehaviorSanitizer and leak checks; the device code is built as usual
and never launched), and run.  Any sanitizer report, or an allocation over its
budget, fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SRC = [os.path.join(ROOT, "dit_dequant_gemm_amd", "csrc", "pd.hip"),
       os.path.join(ROOT, "tests", "host", "pd_search_driver.cpp")]

# host-side instrumentation only: each sanitizer flag follows -Xarch_host
SANITIZERS = {
    "thread": ["-Xarch_host -fsanitize=thread"],
    "address_undefined": ["-Xarch_host -fsanitize=address", "-Xarch_host -fsanitize=undefined",
                          "-Xarch_host -fno-sanitize-recover=all"],
}


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("kind", sorted(SANITIZERS))
def test_pd_search_under_sanitizer(tmp_path, kind):
    exe = str(tmp_path / f"pd_{kind}")
    flags = [f for group in SANITIZERS[kind] for f in group.split()]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++20", *flags,
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "dit_dequant_gemm_amd", "csrc"),
           *SRC, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1", ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-3000:]
    for marker in ("ThreadSanitizer", "AddressSanitizer", "LeakSanitizer", "runtime error:"):
        assert marker not in out, out[-3000:]
    assert "target 7.0" in out
