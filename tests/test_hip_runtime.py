"""The package must leave exactly one HIP runtime in the process.

torch ships its own HIP runtime (requested as libamdhip64.so); libgc links
against libamdhip64.so.7.  Importing the package imports torch before it loads
libgc, so libgc binds to the runtime already mapped.  Loaded the other way
round, the process holds two runtimes and torch's stream handles are invalid
in libgc's (every launch then fails with a HIP error).  Each case runs in a
fresh interpreter so that nothing imported earlier in this process decides it.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "collective_communication_reduction_amd", "libgc.so")

_MAPS = """
paths = set()
with open('/proc/self/maps') as f:
    for line in f:
        if 'libamdhip64' in line:
            paths.add(os.path.realpath(line.split()[-1]))
print(len(paths))
"""


def _runtimes(prelude):
    code = "import os, sys\nsys.path.insert(0, %r)\n" % ROOT + prelude + _MAPS
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert out.returncode == 0, out.stderr
    return int(out.stdout.strip().splitlines()[-1])


def test_package_import_maps_one_hip_runtime():
    assert _runtimes("import collective_communication_reduction_amd\n") == 1


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="two HIP runtimes are only loaded where no GPU is present")
def test_loading_libgc_before_torch_would_map_two():
    # the failure the import order prevents: shows the check above can fail
    assert _runtimes("import ctypes\nctypes.CDLL(%r)\nimport torch\n" % LIB) == 2
