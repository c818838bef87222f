"""bench.py's command-line contract that holds without a GPU (it measures one GPU and says so),
and the host checks of its pattern kernels."""

import os
import subprocess
import sys

import pytest

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


def test_pattern_kernel_refuses_bad_arguments():
    """bench_patterns.hip's host checks (no GPU needed: every call below is refused
    before anything is launched)."""
    import ctypes
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "libbenchpatterns.so")
    if not os.path.exists(path):
        pytest.skip("libbenchpatterns.so is not built")
    lib = ctypes.CDLL(path)
    VPP = ctypes.POINTER(ctypes.c_void_p)
    lib.bp_pattern.restype = ctypes.c_int
    lib.bp_pattern.argtypes = [VPP, ctypes.c_int, VPP, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                               ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    arr = (ctypes.c_void_p * 64)(*([0x10000] * 64))
    sink = ctypes.c_void_p(0x20000)
    cases = [
        (arr, 65, arr, 1, 64, 0, 0, 1),          # too many sources
        (arr, 0, arr, 0, 64, 0, 0, 1),           # nothing to do
        (arr, 1, arr, 1, 0, 0, 0, 1),            # no vectors
        (arr, 1, arr, 1, 64, 0, 2, 1),           # unknown mode
        (arr, 8, arr, 8, 100, 30, 1, 2),         # chunks do not divide the length
        (arr, 8, arr, 6, 64, 8, 1, 2),           # 8 chunks, 6 destinations
        (arr, 8, arr, 8, 64, 8, 1, 5),           # output multiple out of range
    ]
    for src, ns, dst, nd, nvec, cv, mode, om in cases:
        assert lib.bp_pattern(src, ns, dst, nd, nvec, cv, mode, om, sink, None) == 1
    mis = (ctypes.c_void_p * 2)(0x10000, 0x10008)  # second source not 16-byte aligned
    assert lib.bp_pattern(mis, 2, arr, 1, 64, 0, 0, 1, sink, None) == 1
    assert lib.bp_pattern(arr, 1, arr, 1, 64, 0, 0, 1, None, None) == 1   # no sink


def test_committed_profiles_match_the_kernel_sources():
    """Every workload's committed rocprofv3 summary was taken on the current sources of its dominant
    kernel (so bench.py reports its HBM traffic rather than null), and that traffic is the algorithmic
    bytes within 1 %: no kernel re-reads or over-fetches."""
    import re
    sys.path.insert(0, ROOT)
    import bench
    for workload in bench.WORKLOAD_KERNELS:
        assert bench.traffic_from_profiles(workload) is not None, f"{workload}: profile taken on other sources"
        text = open(os.path.join(ROOT, "profiles", f"{workload}_profile.md"), encoding="utf-8").read()
        ratio = float(re.search(r"traffic_over_algorithmic:\s*([0-9.]+)", text).group(1))
        assert 0.99 <= ratio <= 1.01, (workload, ratio)
