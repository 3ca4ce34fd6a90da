"""The host-side ABI checks under AddressSanitizer and UndefinedBehaviorSanitizer.

The C ABI (abi.cpp: validation, workspace layout, dispatch, error reporting)
is built host-only with g++ and -fsanitize=address,undefined, its kernel
launchers replaced by recording stubs (tests/host_abi/stub_launchers.cpp), and
tests/test_abi_host.py runs against that build in a child process with the
ASan runtime preloaded. Any sanitizer report fails the run. No GPU is used.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_activation_linear_amd", "csrc")


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_host_checks_under_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no AddressSanitizer runtime")
    lib = str(tmp_path / "libbitnet_host_sanitized.so")
    cmd = ["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{os.path.join(ROOT, 'include')}", "-shared", "-fPIC", "-g", "-O1",
           "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", os.path.join(CSRC, "abi.cpp"),
           os.path.join(ROOT, "tests", "host_abi", "stub_launchers.cpp"), "-o", lib]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "BITNET_TEST_HOST_LIB": lib,
    })
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_host.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    report = run.stdout[-4000:] + run.stderr[-4000:]
    assert run.returncode == 0, report
    assert "AddressSanitizer" not in report and "runtime error" not in report, report
    assert " passed" in run.stdout and "skipped" not in run.stdout, report
