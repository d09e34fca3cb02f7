"""The C-ABI checks of test_abi_cpu.py on a host-sanitized build of the library.

The build instruments the host code of every source with AddressSanitizer and
UndefinedBehaviorSanitizer (mtp_block_draft_amd/build_sanitized.py); a Python
process that preloads the sanitizer runtime then runs the same argument,
workspace and refusal checks, without a GPU.  Any sanitizer report, or a
failing check, fails this test.  CPU only.
"""
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _builder():
    spec = importlib.util.spec_from_file_location(
        "_dmtp_build_sanitized", os.path.join(ROOT, "mtp_block_draft_amd", "build_sanitized.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.timeout(900)
def test_abi_checks_pass_under_address_and_undefined_behaviour_sanitizers():
    if not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc is not installed")
    b = _builder()
    lib = b.build()
    # the build is instrumented: it calls the sanitizers' report hooks
    if shutil.which("nm"):
        syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, DMTP_ABI_TEST_LIB=lib, LD_PRELOAD=b.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=800)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
