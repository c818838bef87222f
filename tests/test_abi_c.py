"""The C ABI used from plain C: tests/abi_c/abi_demo.c includes gc.h alone,
allocates with hipMalloc, launches on its own HIP stream and checks every
output against closed forms that are exact in any fold order (wrapping int32
sums, small-integer fp32 and bf16 sums averaged over a power of two, and the
placement rules of the data movements), plus refused calls that must leave
their outputs untouched.  build() compiles it; the GPU test runs the binary."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "abi_c", "abi_demo.c")
EXE = os.path.join(ROOT, "tests", "abi_c", "abi_demo")


def test_header_is_plain_c():
    """gc.h and the demo compile as strict C11 (no C++ in the public header; the ROCm
    headers it includes are taken as system headers)."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    p = subprocess.run([cc, "-std=c11", "-fsyntax-only", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}", "-isystem", "/opt/rocm/include", SRC],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stderr[-3000:]


@pytest.mark.gpu
def test_c_program_on_the_gpu():
    assert os.path.exists(EXE), "tests/abi_c/abi_demo is missing: run __graft_entry__.build() first"
    print("running tests/abi_c/abi_demo", flush=True)
    p = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, (p.stdout[-2000:], p.stderr[-3000:])
    assert "checks passed" in p.stdout, p.stdout
