"""The C ABI's host code (argument validation, planning, options, schedule
table: w4_api.cpp) built with AddressSanitizer and UndefinedBehaviorSanitizer
on the host side, running the ABI tests of tests/test_abi.py and the planner
properties of tests/test_plan_properties.py on the CPU (no kernel is
launched).  The sanitized library is loaded through W4_LIBRARY with
the sanitizer runtime preloaded into a child interpreter."""
import os
import subprocess
import sys

import pytest

from mixed_precision_quantized_prepack_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _env(lib_path: str) -> dict:
    return dict(os.environ, LD_PRELOAD=B.sanitizer_runtime(), W4_LIBRARY=lib_path,
                # the interpreter itself is not built for leak checking
                ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


@pytest.fixture(scope="module")
def sanitized_lib():
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc is not available")
    return B.build_sanitized()


def test_sanitized_library_is_the_one_loaded(sanitized_lib):
    code = "import mixed_precision_quantized_prepack_amd as w4; print(w4.lib()._name)"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(sanitized_lib), capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert os.path.samefile(r.stdout.split()[-1], sanitized_lib)
    # the ABI's host code calls into both sanitizers' runtimes
    nm = subprocess.run(["nm", "-D", "--undefined-only", sanitized_lib], capture_output=True, text=True, check=True)
    assert "__asan_report_" in nm.stdout and "__ubsan_handle_" in nm.stdout


def test_abi_tests_pass_under_host_sanitizers(sanitized_lib):
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "tests/test_abi.py",
                        "tests/test_plan_properties.py"],
                       cwd=ROOT, env=_env(sanitized_lib), capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "passed" in out
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer"):
        assert marker not in out, out[-6000:]
