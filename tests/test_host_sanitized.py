"""The host-side tests of libtq (argument validation, the codebook solver,
layout queries, capacity checks) rerun against a build of the library whose
host code runs under AddressSanitizer and UndefinedBehaviorSanitizer (the
device code is built as usual; kv_cache_vector_02_amd.build.
build_host_sanitized), in a child process that preloads the sanitizer
runtime.  Any sanitizer report fails the run."""
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

RUNNER = """
import sys
import kv_cache_vector_02_amd as tq
tq.LIB_PATH = sys.argv[1]
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu", "-k", "not exports",
                      "tests/test_host.py"]))
"""


def test_host_code_under_asan_and_ubsan():
    from kv_cache_vector_02_amd import build as b
    try:
        lib = b.build_host_sanitized()
        runtime = b.asan_runtime()
    except RuntimeError as e:
        pytest.skip(f"no sanitizer build here: {e}")
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", RUNNER, lib], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
