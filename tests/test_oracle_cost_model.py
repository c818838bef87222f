"""The alpha-beta helper reproduces the pages' own estimates (tests/golden/cost_model_numbers.txt)."""

from gen.workloads import llama7b_tensors
from oracle import cost_model as M

GB = 1e9
MiB = 1 << 20


def _want(golden):
    return {l[0]: (float(l[1]), float(l[3])) for l in golden("cost_model_numbers.txt")}


def _close(got, want, rel):
    return abs(got - want) <= rel * abs(want) + 1e-12


def test_page_numbers(golden):
    w = _want(golden)
    got = {
        "ddp7b_traffic_per_gpu": M.ring_allreduce_bytes_per_rank(14 * GB, 8),
        "ddp7b_time": M.ring_allreduce_bytes_per_rank(14 * GB, 8) / (450 * GB),
        "ddp70b_traffic_per_gpu": M.ring_allreduce_bytes_per_rank(140 * GB, 64),
        "ddp70b_time": M.ring_allreduce_bytes_per_rank(140 * GB, 64) / (40 * GB),
        "ar8x64mib_intra_time": M.ring_allreduce_time(64 * MiB, 8, 5e-6, 150 * GB),
        "ar8x64mib_inter_time": M.ring_allreduce_time(64 * MiB, 8, 30e-6, 25 * GB),
        "ar8x64mib_intra_latency": M.ring_allreduce_time(0, 8, 5e-6, 150 * GB),
        "ar8x64mib_inter_latency": M.ring_allreduce_time(0, 8, 30e-6, 25 * GB),
        "ring_vs_naive_ring_factor": M.ring_allreduce_bytes_per_rank(1.0, 8),
        "ring_vs_naive_naive_factor": M.naive_allreduce_bytes(1.0, 8),
        "tp_message_bytes": 4 * 2048 * 4096 * 2,
        "tp_traffic_per_allreduce": M.ring_allreduce_bytes_per_rank(4 * 2048 * 4096 * 2, 8),
        "tp_traffic_per_layer": M.tp_allreduce_bytes_per_step(4, 2048, 4096, 2, 8, 1),
        "tp_traffic_per_step": M.tp_allreduce_bytes_per_step(4, 2048, 4096, 2, 8, 100),
        "tp_time_intra": M.tp_allreduce_bytes_per_step(4, 2048, 4096, 2, 8, 100) / (150 * GB),
        "tp_time_inter": M.tp_allreduce_bytes_per_step(4, 2048, 4096, 2, 8, 100) / (25 * GB),
        "llama7b_params": sum(n for _, n in llama7b_tensors()),
    }
    assert set(got) == set(w)
    for k, v in got.items():
        assert _close(v, w[k][0], w[k][1]), (k, v, w[k])


def test_rs_plus_ag_is_allreduce_traffic():
    for N in (2, 4, 8, 64):
        assert M.ring_rs_or_ag_bytes_per_rank(1000.0, N) * 2 == M.ring_allreduce_bytes_per_rank(1000.0, N)
