"""The host runtime under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU: the library's sources are rebuilt with sanitizers on their host code
only (device code is not instrumented and never runs here) and linked into
tests/sanitize/host_fuzz.cpp, a bounded, seeded fuzz of the checks that run
before any device work: the state-blob parser, resume receipts and scan
metadata.  A sanitizer report, a crash or an unexpected status fails the test.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "streaming_state_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# host-side instrumentation only: each sanitizer flag goes to the host pass
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]


def test_host_runtime_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    from streaming_state_amd import build as lib_build
    srcs = lib_build.sources() + [os.path.join(ROOT, "tests", "sanitize", "host_fuzz.cpp")]
    flags = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC] + SAN

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC] + flags + ["-x", "hip", "-c", src, "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, f"{src}:\n{r.stderr[-3000:]}"
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "host_fuzz")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950"] + SAN[:4] + objs + ["-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe, "200000"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "no failure" in r.stdout
