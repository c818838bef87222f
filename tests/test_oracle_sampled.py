"""Pins the single-element evaluators to the step-by-step ring emulation where both run."""

import numpy as np
import pytest

from oracle import collectives as C
from oracle import sampled as SM
from oracle.numerics import f32_to_bf16


def _inputs(dtype, N, S, rng):
    if dtype == "bf16":
        return [f32_to_bf16(rng.normal(0, 1e-3, size=S).astype(np.float32)) for _ in range(N)]
    if dtype == "fp32":
        return [rng.uniform(-1, 1, size=S).astype(np.float32) for _ in range(N)]
    return [rng.integers(-2**31, 2**31, size=S, dtype=np.int64).astype(np.int32) for _ in range(N)]


@pytest.mark.parametrize("dtype,op", [("bf16", "avg"), ("fp32", "sum"), ("int32", "sum"), ("bf16", "sum")])
@pytest.mark.parametrize("N,S", [(2, 7), (3, 31), (4, 4096), (8, 1001), (16, 300), (64, 640), (5, 3)])
@pytest.mark.parametrize("order", ["ring", "rank"])
def test_all_reduce_at_equals_emulation(dtype, op, N, S, order):
    rng = np.random.default_rng(N * 1000 + S)
    xs = _inputs(dtype, N, S, rng)
    full = C.all_reduce(xs, dtype, op, order)
    pos = np.arange(S)
    vals = np.stack([x[pos] for x in xs])
    got = SM.all_reduce_at(vals, pos, S, dtype, op, order)
    assert np.array_equal(got.view(np.uint8), full[0].view(np.uint8))


@pytest.mark.parametrize("N,rc", [(4, 6), (8, 128), (64, 9)])
@pytest.mark.parametrize("order", ["ring", "rank"])
def test_reduce_scatter_at_equals_emulation(N, rc, order):
    rng = np.random.default_rng(N + rc)
    xs = _inputs("bf16", N, N * rc, rng)
    full = C.reduce_scatter(xs, "bf16", "fp32", "avg", order)
    for j in range(N):
        vals = np.stack([x[j * rc:(j + 1) * rc] for x in xs])
        got = SM.reduce_scatter_at(vals, np.full(rc, j), np.arange(rc), rc, "bf16", "fp32", "avg", order)
        assert np.array_equal(got, full[j])


@pytest.mark.parametrize("tin,tout,op", [("bf16", "fp32", "avg"), ("bf16", "bf16", "avg"), ("fp32", "fp32", "sum"),
                                         ("int32", "int32", "sum")])
@pytest.mark.parametrize("N,rc", [(1, 5), (2, 3), (8, 129), (64, 7)])
@pytest.mark.parametrize("order", ["ring", "rank", "ring_wire"])
def test_reduce_scatter_owner_equals_emulation(tin, tout, op, N, rc, order):
    rng = np.random.default_rng(3 * N + rc)
    xs = _inputs(tin, N, N * rc, rng)
    full = C.reduce_scatter(xs, tin, tout, op, order)
    wire = "bf16" if order == "ring_wire" and tin == "bf16" else None
    for j in range(N):
        got = SM.reduce_scatter_owner([x[j * rc:(j + 1) * rc] for x in xs], j, tin, tout, op, order, wire)
        assert np.array_equal(np.asarray(got).view(np.uint8), np.asarray(full[j]).view(np.uint8)), j


@pytest.mark.parametrize("order", ["ring", "ring_wire"])
def test_reduce_scatter_owner_is_all_reduce_chunk(order):
    # the all-reduce's chunk j (ragged: N does not divide S) is owner j's fold
    N, S = 8, 8 * 50 + 3
    rng = np.random.default_rng(11)
    xs = _inputs("bf16", N, S, rng)
    full = C.all_reduce(xs, "bf16", "avg", order)[0]
    c = -(-S // N)
    for j in range(N):
        lo, hi = min(S, j * c), min(S, (j + 1) * c)
        got = SM.reduce_scatter_owner([x[lo:hi] for x in xs], j, "bf16", "bf16", "avg", order,
                                      "bf16" if order == "ring_wire" else None)
        assert np.array_equal(got, full[lo:hi])
