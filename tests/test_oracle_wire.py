"""Pins for the oracle's wire-faithful bf16 ring (order "ring_wire"): every
message between ranks carries the sender's partial rounded to bf16 (DTLM §11,
low-precision communication with fp32 arithmetic), the receiver adds its own
term in fp32."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import collectives as C
from oracle import fsdp2 as F2
from oracle import sampled as SM
from oracle.numerics import bf16_to_f32, f32_to_bf16


def _b(vals):
    return f32_to_bf16(np.array(vals, dtype=np.float32))


def test_three_rank_worked_example():
    # chunk 0 of 3 one-element chunks is folded ranks 1, 2, 0 with values 1, 2^-8, 2^-8.
    # Wire: rank 2 forwards bf16(1 + 2^-8) = 1 (a tie, to even); the owner adds 2^-8: 1 + 2^-8.
    # fp32 partials: (1 + 2^-8) + 2^-8 = 1 + 2^-7.
    u = 2.0 ** -8
    xs = [_b([u, 0, 0]), _b([1.0, 0, 0]), _b([u, 0, 0])]
    wire = C.reduce_scatter(xs, "bf16", "fp32", "sum", "ring_wire")
    ring = C.reduce_scatter(xs, "bf16", "fp32", "sum", "ring")
    assert float(wire[0][0]) == 1.0 + u and float(ring[0][0]) == 1.0 + 2 * u
    # with a bf16 result the owner's sum 1 + 2^-8 is itself a tie and rounds to 1
    ar = C.all_reduce(xs, "bf16", "sum", "ring_wire")
    assert float(bf16_to_f32(ar[1])[0]) == 1.0
    assert float(bf16_to_f32(C.all_reduce(xs, "bf16", "sum", "ring")[1])[0]) == 1.0 + 2 * u


def test_equal_to_ring_when_no_partial_is_rounded():
    rng = np.random.default_rng(1)
    xs = [_b(rng.normal(size=40)) for _ in range(2)]        # N = 2: the only message is one input
    assert all(np.array_equal(a, b) for a, b in zip(C.all_reduce(xs, "bf16", "avg", "ring_wire"),
                                                     C.all_reduce(xs, "bf16", "avg", "ring")))
    ys = [rng.normal(size=40).astype(np.float32) for _ in range(5)]   # fp32 data travels unrounded
    assert all(np.array_equal(a, b) for a, b in zip(C.all_reduce(ys, "fp32", "sum", "ring_wire"),
                                                     C.all_reduce(ys, "fp32", "sum", "ring")))


@pytest.mark.parametrize("N", [8, 64])
def test_error_bound_and_size(N):
    """|wire - exact| <= (N - 1) * (2^-8 + 2^-24) * sum|x| elementwise (each of the
    N - 2 rounded messages and N - 1 fp32 adds errs by at most its unit roundoff
    times a partial bounded by sum|x|); and the wire ring's error is the larger one."""
    rng = np.random.default_rng(N)
    S = 4 * N
    xs = [_b(rng.normal(scale=1e-3, size=S)) for _ in range(N)]
    wide = [bf16_to_f32(x).astype(np.float64) for x in xs]
    ys_w = C.ring_reduce_scatter_partials(xs, "bf16", wire="bf16")
    ys_r = C.ring_reduce_scatter_partials(xs, "bf16")
    c = S // N
    err_w = err_r = Fraction(0)
    for j in range(N):
        for k in range(c):
            e = j * c + k
            exact = sum(Fraction(float(w[e])) for w in wide)
            mag = sum(abs(Fraction(float(w[e]))) for w in wide)
            dw = abs(Fraction(float(ys_w[j][k])) - exact)
            dr = abs(Fraction(float(ys_r[j][k])) - exact)
            assert dw <= (N - 1) * (Fraction(1, 2**8) + Fraction(1, 2**24)) * mag
            err_w += dw
            err_r += dr
    assert err_w > 100 * err_r


@pytest.mark.parametrize("N,S", [(4, 16), (8, 29), (64, 130)])
def test_sampled_evaluation_matches_emulation(N, S):
    rng = np.random.default_rng(S)
    xs = [_b(rng.normal(size=S)) for _ in range(N)]
    full = C.all_reduce(xs, "bf16", "avg", "ring_wire")
    pos = np.arange(S)
    vals = np.stack([x[pos] for x in xs])
    assert np.array_equal(SM.all_reduce_at(vals, pos, S, "bf16", "avg", "ring_wire"), full[0])
    rs = C.reduce_scatter([x[:N * (S // N)] for x in xs], "bf16", "fp32", "avg", "ring_wire")
    rc = S // N
    for j in range(N):
        got = SM.reduce_scatter_at(np.stack([x[j * rc:(j + 1) * rc] for x in xs]), np.full(rc, j), np.arange(rc),
                                   rc, "bf16", "fp32", "avg", "ring_wire")
        assert np.array_equal(got, rs[j])


def test_fsdp2_wire_matches_flat_when_rows_divide():
    rng = np.random.default_rng(5)
    N, rows, cols = 4, [8, 4], [3, 5]
    grads = [[_b(rng.normal(size=r * c)) for r, c in zip(rows, cols)] for _ in range(N)]
    out = F2.reduce_scatter(grads, rows, cols, "bf16", "bf16", "avg", "ring_wire")
    for p in range(len(rows)):
        flat = C.reduce_scatter([grads[i][p] for i in range(N)], "bf16", "bf16", "avg", "ring_wire")
        assert all(np.array_equal(out[j][p], flat[j]) for j in range(N))
