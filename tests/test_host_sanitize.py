"""The C ABI's host layer (argument validation, aliasing rules, chunk / bucket /
all-to-all / routing planning in api.cpp) built for the host with
AddressSanitizer and UndefinedBehaviorSanitizer, linked against launch stubs,
and driven by a seeded argument fuzz (tests/sanitize/abi_fuzz.cpp) with the
library's GC_DEBUG plan-table checks switched on: no sanitizer report, no
launch after a refused call, every launch inside the buffers the contract gives
the caller, no plan-table check firing, and every entry point both accepted and
refused some calls.  No GPU is involved."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "tests", "sanitize", "build.sh")


@pytest.fixture(scope="module")
def fuzzer(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ is not available")
    exe = str(tmp_path_factory.mktemp("sanitize") / "abi_fuzz")
    p = subprocess.run(["bash", BUILD, exe], capture_output=True, text=True, timeout=600)
    assert p.returncode == 0, p.stderr[-4000:]
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_abi_fuzz_under_asan_and_ubsan(fuzzer, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([fuzzer, "30000", str(seed)], capture_output=True, text=True, timeout=600, env=env)
    assert p.returncode == 0, (p.stdout[-2000:], p.stderr[-4000:])
    assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr, p.stderr[-4000:]
    assert "GC_DEBUG" not in p.stderr, p.stderr[-4000:]        # the library's plan-table checks held
    assert ", 0 failures" in p.stdout, p.stdout[-2000:]
