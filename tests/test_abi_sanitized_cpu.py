"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is built a second time with the host code instrumented (the device code
unchanged), and the host-side ABI tests (`test_abi_cpu.py`: validation of every entry
point before any device call, the packed-header format and its rejections, sizes,
status strings) run against it in a child process that preloads the ASan runtime.
Any sanitizer report ends the child with an error; the test requires a clean exit.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized_library(tmp_path_factory):
    from w4a16_int4_weight_amd import build
    out = str(tmp_path_factory.mktemp("asan") / "libw4a16_asan.so")
    try:
        build.build(out=out, sanitize_host=True)
        runtime = build.asan_runtime()
    except RuntimeError as e:           # no ROCm compiler on this host
        pytest.skip(f"host-sanitized build unavailable: {e}")
    return out, runtime


def test_abi_host_code_is_clean_under_asan_and_ubsan(sanitized_library):
    lib, runtime = sanitized_library
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime,
        "W4A16_LIBRARY": lib,
        # the interpreter itself is not instrumented: its allocations are not leaks of ours
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                          "-q", "-x", "-s", "-p", "no:cacheprovider"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
