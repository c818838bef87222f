"""Pins for the oracle's two-level all-reduce and HSDP reduce-scatter (AIG6
Table 6-2 hierarchical all-reduce, AIG6 §6.3.6 HSDP on 2 nodes x 8 GPUs, DTLM
§4 HSDP mesh): exact sums, reductions to the flat ring when one level is
trivial, a fold-order case worked by hand, and the HSDP shards as slices of
the all-reduce."""

import numpy as np
import pytest

from oracle import collectives as C
from oracle import hierarchical as H
from oracle.numerics import f32_to_bf16


def _ints(rng, N, S):
    return [rng.integers(-2**31, 2**31, size=S).astype(np.int32) for _ in range(N)]


@pytest.mark.parametrize("R,S,count", [(2, 8, 1000), (2, 2, 7), (4, 3, 50), (3, 4, 5), (8, 8, 130), (2, 1, 9)])
@pytest.mark.parametrize("order", ["ring", "rank"])
def test_exact_int32_sums(R, S, count, order):
    rng = np.random.default_rng(R * 10 + S)
    xs = _ints(rng, R * S, count)
    out = H.all_reduce(xs, S, "int32", "sum", order)
    total = [sum(int(x[e]) for x in xs) % 2**32 for e in range(count)]
    total = np.array([t - 2**32 if t >= 2**31 else t for t in total], dtype=np.int32)
    assert all(np.array_equal(o, total) for o in out)


@pytest.mark.parametrize("N,count", [(4, 4 * 37 + 3), (8, 100), (3, 2)])
@pytest.mark.parametrize("dtype,op", [("bf16", "avg"), ("fp32", "sum")])
def test_one_trivial_level_is_the_flat_ring(N, count, dtype, op):
    rng = np.random.default_rng(N + count)
    x32 = [rng.normal(size=count).astype(np.float32) for _ in range(N)]
    xs = [f32_to_bf16(x) for x in x32] if dtype == "bf16" else x32
    flat = C.all_reduce(xs, dtype, op, "ring")
    for S in (N, 1):                     # one group of N, or N groups of one
        got = H.all_reduce(xs, S, dtype, op, "ring")
        assert all(np.array_equal(g, f) for g, f in zip(got, flat)), S


def test_fold_order_worked_example():
    # R = S = 2, one element per rank: ranks (0,0), (0,1), (1,0), (1,1) hold 1, 1, 2^24, -2^24.
    # Level one folds each group from member 1: group 0 gives 1 + 1 = 2, group 1 gives -2^24 + 2^24 = 0.
    # Level two folds the groups from group 1: 0 + 2 = 2, exact.  The flat ring over 4 ranks folds
    # ranks 1, 2, 3, 0: ((1 + 2^24) - 2^24) + 1 = 1, since 1 + 2^24 rounds to 2^24 in fp32.
    big = 2.0 ** 24
    xs = [np.array([v], np.float32) for v in (1.0, 1.0, big, -big)]
    assert float(H.all_reduce(xs, 2, "fp32", "sum", "ring")[0][0]) == 2.0
    assert float(C.all_reduce(xs, "fp32", "sum", "ring")[0][0]) == 1.0
    # rank order at both levels with 1, 2^24, 1, -2^24: group 0 gives 1 + 2^24 = 2^24 (a tie, to even),
    # group 1 gives 1 - 2^24 exactly, and 2^24 + (1 - 2^24) = 1; the flat rank order gives
    # ((1 + 2^24) + 1) - 2^24 = 0
    ys = [np.array([v], np.float32) for v in (1.0, big, 1.0, -big)]
    assert float(H.all_reduce(ys, 2, "fp32", "sum", "rank")[0][0]) == 1.0
    assert float(C.all_reduce(ys, "fp32", "sum", "rank")[0][0]) == 0.0


@pytest.mark.parametrize("R,S,rc", [(2, 8, 33), (4, 2, 5), (3, 3, 1), (2, 4, 0)])
@pytest.mark.parametrize("order", ["ring", "rank"])
def test_hsdp_shards_are_slices_of_the_all_reduce(R, S, rc, order):
    rng = np.random.default_rng(R * S + rc)
    xs = [f32_to_bf16(rng.normal(size=S * rc).astype(np.float32)) for _ in range(R * S)]
    full = H.all_reduce(xs, S, "bf16", "avg", order)[0]
    sh = H.hsdp_reduce_scatter(xs, S, "bf16", "bf16", "avg", order)
    for g in range(R):
        for i in range(S):
            assert np.array_equal(sh[g * S + i], full[i * rc:(i + 1) * rc])


def test_avg_divides_by_all_ranks_once():
    # avg over N = 6 ranks of dyadic values: exact mean, not a mean of group means re-divided
    xs = [np.full(6, float(v), np.float32) for v in (1, 2, 3, 4, 5, 9)]
    out = H.all_reduce(xs, 3, "fp32", "avg", "ring")
    assert np.all(out[0] == np.float32(24 / 6))
    sh = H.hsdp_reduce_scatter(xs, 3, "fp32", "fp32", "avg", "ring")
    assert all(np.all(s == np.float32(4.0)) for s in sh)


def test_group_size_must_divide():
    with pytest.raises(ValueError):
        H.all_reduce([np.zeros(3, np.float32)] * 6, 4, "fp32")
    with pytest.raises(ValueError):
        H.hsdp_reduce_scatter([np.zeros(3, np.float32)] * 4, 2, "fp32")


@pytest.mark.parametrize("R,S,count", [(2, 8, 301), (4, 3, 50), (3, 4, 7), (2, 2, 1), (2, 8, 320), (4, 3, 51)])
@pytest.mark.parametrize("order", ["ring", "rank"])
def test_sampled_two_level_matches_emulation(R, S, count, order):
    from oracle import sampled as SM
    rng = np.random.default_rng(R + S + count)
    xs = [f32_to_bf16(rng.normal(size=count).astype(np.float32)) for _ in range(R * S)]
    full = H.all_reduce(xs, S, "bf16", "avg", order)[0]
    pos = np.arange(count)
    g0, m0 = SM.hier_fold_starts(pos, count, S, R, order)
    got = SM.hier_reduce_positions(np.stack([x[pos] for x in xs]), S, g0, m0, "bf16", "avg", "bf16")
    assert np.array_equal(got, full)
    if count % S == 0:
        rc = count // S
        sh = H.hsdp_reduce_scatter(xs, S, "bf16", "fp32", "avg", order)
        g0, m0 = SM.hier_fold_starts(pos, count, S, R, order, chunk=rc)
        got = SM.hier_reduce_positions(np.stack([x[pos] for x in xs]), S, g0, m0, "bf16", "avg", "fp32")
        assert np.array_equal(got, np.concatenate([sh[i] for i in range(S)]))


# ---------------------------------------------------------------- bf16 on the wire

@pytest.mark.parametrize("N,count", [(4, 4 * 37 + 3), (8, 100), (3, 2)])
def test_wire_one_trivial_level_is_the_flat_wire_ring(N, count):
    rng = np.random.default_rng(7 * N + count)
    xs = [f32_to_bf16(rng.normal(size=count).astype(np.float32)) for _ in range(N)]
    flat = C.all_reduce(xs, "bf16", "avg", "ring_wire")
    for S in (N, 1):                     # one group of N, or N groups of one
        got = H.all_reduce(xs, S, "bf16", "avg", "ring_wire")
        assert all(np.array_equal(g, f) for g, f in zip(got, flat)), S


def test_wire_worked_example():
    # R = S = 2, one element per rank, bf16 bits: ranks (0,0), (0,1), (1,0), (1,1) hold 0, 2^-8, 2^-8, 1.
    # Group 1 folds from member 1: 1 + 2^-8 (fp32, exact).  Group 0: 2^-8 + 0 = 2^-8.
    # Across groups the fold starts at group 1, whose partial goes on the wire as bf16:
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 and rounds to even, 1; group 0 adds 2^-8 -> 1 + 2^-8,
    # whose bf16 output (sum) is again the tie -> 1.0.  With fp32 partials the sum is 1 + 2^-7 exactly.
    # The flat wire ring over the four ranks folds 2^-8, 2^-8, 1, 0 and never rounds: 1 + 2^-7.
    one, eps, zero = 0x3F80, 0x3B80, 0x0000
    xs = [np.array([b], np.uint16) for b in (zero, eps, eps, one)]
    assert int(H.all_reduce(xs, 2, "bf16", "sum", "ring_wire")[0][0]) == 0x3F80
    assert int(H.all_reduce(xs, 2, "bf16", "sum", "ring")[0][0]) == 0x3F81
    assert int(C.all_reduce(xs, "bf16", "sum", "ring_wire")[0][0]) == 0x3F81
    # the HSDP shard (one element per member chunk: count 2, chunk 0 holds element 0) sees the same rounding
    ys = [np.array([b, zero], np.uint16) for b in (zero, eps, eps, one)]
    sh = H.hsdp_reduce_scatter(ys, 2, "bf16", "fp32", "sum", "ring_wire")
    assert float(sh[0][0]) == 1.0 + 2.0 ** -8 and float(sh[2][0]) == 1.0 + 2.0 ** -8
    assert float(H.hsdp_reduce_scatter(ys, 2, "bf16", "fp32", "sum", "ring")[0][0]) == 1.0 + 2.0 ** -7


@pytest.mark.parametrize("R,S,count", [(2, 8, 130), (4, 3, 50)])
def test_wire_changes_nothing_for_fp32_data(R, S, count):
    rng = np.random.default_rng(R + S)
    xs = [rng.normal(size=count).astype(np.float32) for _ in range(R * S)]
    a = H.all_reduce(xs, S, "fp32", "sum", "ring_wire")[0]
    b = H.all_reduce(xs, S, "fp32", "sum", "ring")[0]
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("R,S,count", [(2, 8, 301), (4, 3, 50), (3, 4, 7), (2, 2, 1), (2, 8, 320)])
@pytest.mark.parametrize("order", ["ring", "rank", "ring_wire"])
def test_block_evaluator_matches_emulation(R, S, count, order):
    # each cell (chunk i, cross-group piece h) folded as one block with its fold start
    from oracle import sampled as SM
    rng = np.random.default_rng(R * S + count)
    xs = [f32_to_bf16(rng.normal(size=count).astype(np.float32)) for _ in range(R * S)]
    full = H.all_reduce(xs, S, "bf16", "avg", order)[0]
    wire = "bf16" if order == "ring_wire" else None
    c1 = -(-count // S)
    got = np.empty(count, np.uint16)
    for i in range(S):
        lo, hi = min(count, i * c1), min(count, (i + 1) * c1)
        c2 = max(1, -(-(hi - lo) // R))
        for h in range(R):
            a, b = lo + min(hi - lo, h * c2), lo + min(hi - lo, (h + 1) * c2)
            if a == b:
                continue
            g0, m0 = ((h + 1) % R, (i + 1) % S) if order != "rank" else (0, 0)
            got[a:b] = SM.hier_reduce_block([x[a:b] for x in xs], S, g0, m0, "bf16", "avg", "bf16", wire)
    assert np.array_equal(got, full)
