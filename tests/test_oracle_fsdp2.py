"""Pins for the oracle's FSDP2 per-parameter Shard(0) reduce-scatter and
all-gather (DTLM §4 FSDP2): the pages' worked examples, uneven and empty
shards, exact sums and the ring's fold order."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import collectives as C
from oracle import fsdp2 as F2
from oracle.numerics import bf16_to_f32, f32_to_bf16


def _unit1(golden):
    lines = golden("fsdp2_unit1.txt")
    params = [(l[1], int(l[2]), int(l[3])) for l in lines if l[0] == "param"]
    world = int(next(l[1] for l in lines if l[0] == "world"))
    return lines, params, world


def test_unit1_shards(golden):
    lines, params, world = _unit1(golden)
    names = [p[0] for p in params]
    for l in lines:
        if l[0] == "shard":
            p = names.index(l[1])
            _, rows, cols = params[p]
            r, lo, hi = int(l[2]), int(l[3]), int(l[4])
            assert F2.shard_elems(rows, cols, world)[r] == (lo * cols, hi * cols)


def test_uneven_and_empty_shards(golden):
    lines = golden("uneven_shards.txt")
    cur = None
    for l in lines:
        if l[0] == "case":
            cur = (int(l[1]), int(l[2]))
        else:
            r, lo, hi = int(l[1]), int(l[2]), int(l[3])
            assert F2.shard_elems(cur[0], 3, cur[1])[r] == (3 * lo, 3 * hi)   # the pages' [rows, 3] weights


def test_unit1_reduce_scatter_example(golden):
    """x_{j,i} = rank i's gradient of row j; rank j keeps x_j0 + x_j1."""
    lines, params, world = _unit1(golden)
    rows = [p[1] for p in params]
    cols = [p[2] for p in params]
    grads = [[np.array([100 * j + 10 * i + c for j in range(rows[p]) for c in range(cols[p])], np.int32)
              for p in range(len(params))] for i in range(world)]
    out = F2.reduce_scatter(grads, rows, cols, "int32")
    names = [p[0] for p in params]
    for l in lines:
        if l[0] == "rs":
            p, r, j = names.index(l[1]), int(l[2]), int(l[3])
            want = [sum(100 * j + 10 * i + c for i in range(world)) for c in range(cols[p])]
            assert list(out[r][p]) == want
    full = F2.all_gather(out, rows, cols, "int32")
    for d in range(world):
        for p in range(len(params)):
            want = [sum(100 * j + 10 * i + c for i in range(world)) for j in range(rows[p]) for c in range(cols[p])]
            assert list(full[d][p]) == want


@pytest.mark.parametrize("N,rows,cols", [(4, [2, 3, 9, 1], [3, 5, 1, 7]), (3, [1, 10, 4], [4, 2, 6]),
                                         (8, [5, 17, 64], [3, 2, 1]), (1, [3], [2])])
def test_reduce_scatter_exact_int32_and_empty_shards(N, rows, cols):
    rng = np.random.default_rng(N)
    grads = [[rng.integers(-2**31, 2**31, size=r * c).astype(np.int32) for r, c in zip(rows, cols)]
             for _ in range(N)]
    out = F2.reduce_scatter(grads, rows, cols, "int32", order="ring")
    for p, (r_, c_) in enumerate(zip(rows, cols)):
        total = [sum(int(grads[i][p][e]) for i in range(N)) % 2**32 for e in range(r_ * c_)]
        total = [t - 2**32 if t >= 2**31 else t for t in total]
        c_rows = -(-r_ // N)
        for j in range(N):
            lo, hi = min(r_, j * c_rows) * c_, min(r_, (j + 1) * c_rows) * c_
            assert list(out[j][p]) == total[lo:hi]
            if lo == hi:
                assert out[j][p].size == 0                      # trailing ranks hold empty shards
    full = F2.all_gather(out, rows, cols, "int32")
    assert all(np.array_equal(full[d][p], full[0][p]) for d in range(N) for p in range(len(rows)))


def test_ring_fold_order_per_parameter():
    # one row per rank; chunk 0 is folded from rank 1: ((1 + 1) - 2^24) + 2^24 = 2 exactly,
    # while the rank order gives ((2^24 + 1) + 1) - 2^24 = 0 in fp32
    big = np.float32(2.0 ** 24)
    vals = [big, 1.0, 1.0, -big]
    grads = [[np.full(4, vals[i], np.float32)] for i in range(4)]
    ring = F2.reduce_scatter(grads, [4], [1], "fp32", order="ring")
    rank = F2.reduce_scatter(grads, [4], [1], "fp32", order="rank")
    assert float(ring[0][0][0]) == 2.0 and float(rank[0][0][0]) == 0.0
    assert float(ring[3][0][0]) == 0.0                            # chunk 3: ranks 0, 1, 2, 3


def test_reduce_scatter_avg_bf16_to_fp32_within_summation_bound():
    """Each averaged fp32 value lies within the recursive-summation bound of the
    exact mean: |fl(sum)/N * N - sum| <= N * 2^-24 * sum|x| (Higham §4.2, plus
    one rounding for the division)."""
    rng = np.random.default_rng(3)
    N, rows, cols = 5, [7, 2], [3, 11]
    grads = [[f32_to_bf16(rng.normal(size=r * c).astype(np.float32)) for r, c in zip(rows, cols)]
             for _ in range(N)]
    out = F2.reduce_scatter(grads, rows, cols, "bf16", "fp32", op="avg")
    for p, (r_, c_) in enumerate(zip(rows, cols)):
        vals = [bf16_to_f32(grads[i][p]).astype(np.float64) for i in range(N)]
        for j, (lo, hi) in enumerate(F2.shard_elems(r_, c_, N)):
            assert out[j][p].dtype == np.float32 and out[j][p].size == hi - lo
            for e in range(lo, hi):
                exact = sum(Fraction(float(v[e])) for v in vals)
                mag = sum(abs(Fraction(float(v[e]))) for v in vals)
                got = Fraction(float(out[j][p][e - lo])) * N
                assert abs(got - exact) <= Fraction(101, 100) * N * mag / 2**24


def test_matches_flat_reduce_scatter_when_rows_divide():
    """With N dividing every parameter's rows, each parameter's reduce-scatter
    equals the flat reduce-scatter of that parameter alone."""
    rng = np.random.default_rng(4)
    N, rows, cols = 4, [8, 4], [3, 5]
    grads = [[f32_to_bf16(rng.normal(size=r * c).astype(np.float32)) for r, c in zip(rows, cols)]
             for _ in range(N)]
    out = F2.reduce_scatter(grads, rows, cols, "bf16", "bf16", op="avg")
    for p in range(len(rows)):
        flat = C.reduce_scatter([grads[i][p] for i in range(N)], "bf16", "bf16", op="avg")
        for j in range(N):
            assert np.array_equal(out[j][p], flat[j])


def test_all_gather_rejects_wrong_shard_sizes():
    with pytest.raises(ValueError):
        F2.all_gather([[np.zeros(3, np.float32)], [np.zeros(3, np.float32)]], [3], [2], "fp32")
