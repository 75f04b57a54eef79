"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

fa_api.cpp (argument validation, launch planning, workspace layouts, the
compute-unit query) is compiled with g++ -fsanitize=address,undefined
together with stand-ins for the kernel launchers and the three HIP runtime
calls it makes (tests/sanitize/launch_stubs.cpp), and driven by
tests/sanitize/host_checks.cpp: every entry point with invalid arguments
(null, shapes up to INT_MAX, strides, alignment, aliasing, mask layouts,
dropout probabilities), valid arguments with fake device addresses (never
dereferenced), the planner's choices at 256 and at 304 compute units, and
the once-per-device caching of that count.  A sanitizer report or a failed
check fails the test.  Host code only: no GPU code is built here.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")


def _gxx():
    return shutil.which("g++")


@pytest.mark.skipif(_gxx() is None, reason="g++ not available")
def test_host_abi_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_checks")
    cmd = [_gxx(), "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "tiled_attention_15_amd", "csrc"),
           "-I" + SAN, os.path.join(ROOT, "tiled_attention_15_amd", "csrc", "fa_api.cpp"),
           os.path.join(SAN, "launch_stubs.cpp"), os.path.join(SAN, "host_checks.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and ("asan" in r.stderr.lower() or "ubsan" in r.stderr.lower()) and \
            "cannot find" in r.stderr:
        pytest.skip("sanitizer runtime not installed: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "host checks passed" in run.stdout
