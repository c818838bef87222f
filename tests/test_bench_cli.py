"""bench.py's command-line contract that holds without a GPU: it measures one GPU and says so."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "--gpus 2" in p.stderr and "one GPU" in p.stderr
    assert p.stdout == ""


def test_every_workload_has_a_kernel_source_list():
    sys.path.insert(0, ROOT)
    import bench
    for w in bench.WORKLOAD_KERNELS:
        for rel in bench.KERNEL_SOURCES[bench.WORKLOAD_KERNELS[w]]:
            assert os.path.exists(os.path.join(ROOT, rel)), rel
        assert len(bench.kernel_hash(w)) == 16
