"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The argument checks, split planning and workspace sizing of abi.hip are
rebuilt with both sanitizers (device code unchanged) into libmla_san.so, and
the host-side ABI tests run against that build in a fresh process with the
sanitizer runtime preloaded.  Any report (an out-of-bounds access, an
overflow, a misaligned or null access) aborts that process, so the test
passes only if every host check runs clean.  No GPU is used.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc_available():
    from mla_latent_kv_36_amd import build
    try:
        build.hipcc()
        return True
    except RuntimeError:
        return False


@pytest.mark.skipif(not _hipcc_available(), reason="hipcc is needed to build the sanitized library")
def test_host_abi_checks_run_clean_under_asan_and_ubsan():
    from mla_latent_kv_36_amd import build
    lib = build.build_sanitized()
    env = dict(os.environ)
    env.update({
        "MLA_LIBRARY": lib,
        "LD_PRELOAD": build.sanitizer_runtime(),
        # leaks of the interpreter and the HIP runtime are not this library's
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout
