"""Pins for the oracle's ring reduce-scatter / all-gather / all-reduce.

Each pin is independent of the oracle's own code: the pages' worked N = 4
schedules (tests/golden), closed-form traffic, exact rational sums, Python
big-integer sums, and a constructed cancellation case that only the ring's fold
order gets right.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import collectives as C
from oracle.numerics import bf16_to_f32, f32_to_bf16


def _parse_terms(s):
    return tuple(int(t) for t in s.split(","))


# ------------------------------------------------------------- worked examples

def test_reduce_scatter_schedule_matches_worked_example(golden):
    lines = golden("ring_reduce_scatter_n4.txt")
    want_msgs = [(int(a), int(b), int(c), int(d), _parse_terms(e)) for k, a, b, c, d, e in
                 (l for l in lines if l[0] == "msg")]
    want_final = {int(o): _parse_terms(t) for k, o, t in (l for l in lines if l[0] == "final")}
    # tag x_{j,i} = 2^(4j+i): every partial sum names its terms exactly
    xs = [np.array([1 << (4 * j + i) for j in range(4)], dtype=np.int32) for i in range(4)]
    tr = C.RingTrace(4)
    ys = C.ring_reduce_scatter_partials(xs, "int32", trace=tr)
    got = sorted((m.step, m.src, m.dst, m.chunk, m.terms) for m in tr.messages)
    assert got == sorted(want_msgs)
    for m in tr.messages:                       # every message's value is the sum of its terms
        assert m.elems == 1
    for j in range(4):
        assert int(ys[j][0]) == sum(1 << (4 * j + i) for i in want_final[j])
        assert want_final[j][-1] == j           # the last hop lands on the owner
    assert tr.steps == 3


def test_all_gather_schedule_matches_worked_example(golden):
    lines = golden("ring_all_gather_n4.txt")
    want_msgs = sorted((int(a), int(b), int(c), int(d)) for k, a, b, c, d in (l for l in lines if l[0] == "msg"))
    tr = C.RingTrace(4)
    shards = [np.array([100 + k], dtype=np.int32) for k in range(4)]
    out = C.ring_all_gather(shards, trace=tr)
    got = sorted((m.step, m.src, m.dst, m.chunk) for m in tr.messages)
    assert got == want_msgs
    # holdings in arrival order after each step, rebuilt from the message log
    arrivals = {r: [r] for r in range(4)}
    for step in (1, 2, 3):
        for m in sorted(tr.messages, key=lambda m: (m.step, m.src)):
            if m.step == step:
                arrivals[m.dst].append(m.chunk)
        for k, st, r, seq in (l for l in lines if l[0] == "hold"):
            if int(st) == step:
                assert tuple(arrivals[int(r)]) == _parse_terms(seq)
    for k, r, seq in (l for l in lines if l[0] == "final"):
        assert [int(v) - 100 for v in out[int(r)]] == list(_parse_terms(seq))


def test_fold_order_is_the_rings():
    # chunk 0 terms in ring order: x01 = 2^24, x02 = 1, x03 = 1, x00 = -2^24.
    # Ring: ((2^24 + 1) + 1) - 2^24 = 0 in fp32; rank order: ((-2^24 + 2^24) + 1) + 1 = 2.
    big = np.float32(2.0 ** 24)
    xs = [np.array([-big, 0, 0, 0], np.float32), np.array([big, 0, 0, 0], np.float32),
          np.array([1, 0, 0, 0], np.float32), np.array([1, 0, 0, 0], np.float32)]
    ring = C.all_reduce(xs, "fp32", "sum", "ring")
    rank = C.all_reduce(xs, "fp32", "sum", "rank")
    assert all(r[0] == 0.0 for r in ring)
    assert all(r[0] == 2.0 for r in rank)
    # the same data rotated into chunk 2 (owner 2, first term from rank 3)
    S = 4
    xs2 = [np.zeros(S, np.float32) for _ in range(4)]
    for i, v in zip([3, 0, 1, 2], [big, 1, 1, -big]):
        xs2[i][2] = v
    assert C.all_reduce(xs2, "fp32", "sum", "ring")[0][2] == 0.0


def test_first_operand_starts_the_fold():
    # -0.0 + -0.0 + ... stays -0.0 only when the fold starts from the first term
    xs = [np.array([-0.0, -0.0], np.float32) for _ in range(3)]
    for order in ("ring", "rank"):
        out = C.all_reduce(xs, "fp32", "sum", order)
        assert np.all(np.signbit(out[0]))


# ------------------------------------------------------------- brute force

def _exact_f32(fr):
    """Round an exact rational to fp32, nearest-even, by bracketing with np.nextafter (brute force)."""
    approx = np.float32(float(fr))
    cands = {approx, np.nextafter(approx, np.float32(np.inf)), np.nextafter(approx, np.float32(-np.inf))}
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("S", [0, 1, 3, 7, 8, 16, 29])
def test_exactly_summable_fp32_equals_exact_sum(N, S):
    rng = np.random.default_rng(N * 100 + S)
    # small integers times a common power of two: every partial sum is exact in fp32
    xs = [(rng.integers(-1000, 1000, size=S).astype(np.float32) * np.float32(2.0 ** -7)) for _ in range(N)]
    for order in ("ring", "rank"):
        out = C.all_reduce(xs, "fp32", "sum", order)
        for r in range(N):
            assert len(out[r]) == S
            for e in range(S):
                assert Fraction(float(out[r][e])) == C.exact_sum(x[e] for x in xs)
        avg = C.all_reduce(xs, "fp32", "avg", order)
        for e in range(S):
            want = _exact_f32(C.exact_sum(x[e] for x in xs) / N)
            assert avg[0][e] == want


@pytest.mark.parametrize("N,S", [(2, 9), (3, 10), (4, 4), (7, 50), (8, 64)])
def test_int32_wraps_like_big_integer_sum(N, S):
    rng = np.random.default_rng(S)
    xs = [rng.integers(-2**31, 2**31, size=S, dtype=np.int64).astype(np.int32) for _ in range(N)]
    out = C.all_reduce(xs, "int32", "sum", "ring")
    for e in range(S):
        total = sum(int(x[e]) for x in xs) % (1 << 32)
        want = total - (1 << 32) if total >= (1 << 31) else total
        assert all(int(o[e]) == want for o in out)


@pytest.mark.parametrize("N", [2, 4, 8, 16, 64])
def test_random_fp32_within_recursive_summation_bound(N):
    S = 3 * N + 5
    rng = np.random.default_rng(N)
    xs = [rng.uniform(-1, 1, size=S).astype(np.float32) for _ in range(N)]
    u = Fraction(1, 1 << 24)
    out = C.all_reduce(xs, "fp32", "sum", "ring")[0]
    for e in range(S):
        exact = C.exact_sum(x[e] for x in xs)
        mag = sum(abs(Fraction(float(x[e]))) for x in xs)
        bound = (N - 1) * u * mag * (1 + N * u)   # Higham, recursive summation, first-order term + slack
        assert abs(Fraction(float(out[e])) - exact) <= bound


def test_bf16_average_rounds_fp32_mean():
    N, S = 8, 40
    rng = np.random.default_rng(3)
    xs = [f32_to_bf16(rng.normal(0, 1e-3, size=S).astype(np.float32)) for _ in range(N)]
    out = C.all_reduce(xs, "bf16", "avg", "ring")
    chunks = C.owner_chunks(S, N)
    for j, (lo, hi) in enumerate(chunks):
        for e in range(lo, hi):
            acc = None
            for t in range(1, N + 1):            # ring order j+1, ..., j written out by hand
                v = bf16_to_f32(xs[(j + t) % N][e:e + 1])[0]
                acc = v if acc is None else np.float32(acc + v)
            want = f32_to_bf16(np.float32(acc / np.float32(N)))
            assert all(o[e] == want for o in out)


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("N,S", [(4, 16), (8, 64), (3, 10), (5, 3), (8, 0), (1, 7)])
def test_ring_traffic_closed_form(N, S):
    xs = [np.ones(S, np.float32) for _ in range(N)]
    tr = C.RingTrace(N)
    C.all_reduce(xs, "fp32", "sum", "ring", trace=tr)
    chunks = C.owner_chunks(S, N)
    size = [hi - lo for lo, hi in chunks]
    for r in range(N):
        want = (S - size[r]) + (S - size[(r + 1) % N]) if N > 1 else 0
        assert tr.sent_elems[r] == want
        if S % N == 0:
            assert tr.sent_elems[r] == 2 * (N - 1) * S // N
    assert tr.steps == 2 * (N - 1)


def test_owner_chunks_rule():
    assert C.owner_chunks(10, 4) == [(0, 3), (3, 6), (6, 9), (9, 10)]
    assert C.owner_chunks(2, 4) == [(0, 1), (1, 2), (2, 2), (2, 2)]
    assert C.owner_chunks(0, 3) == [(0, 0)] * 3
    for S in range(0, 40):
        for N in range(1, 9):
            ch = C.owner_chunks(S, N)
            assert ch[0][0] == 0 and ch[-1][1] == S
            assert all(a[1] == b[0] for a, b in zip(ch, ch[1:]))


# ------------------------------------------------------------- invariants

@pytest.mark.parametrize("dtype,op", [("fp32", "sum"), ("bf16", "avg"), ("int32", "sum"), ("fp32", "avg")])
@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_all_reduce_is_reduce_scatter_then_all_gather(dtype, op, N):
    S = N * 11
    rng = np.random.default_rng(N)
    if dtype == "int32":
        xs = [rng.integers(-1000, 1000, size=S).astype(np.int32) for _ in range(N)]
    elif dtype == "bf16":
        xs = [f32_to_bf16(rng.normal(size=S).astype(np.float32)) for _ in range(N)]
    else:
        xs = [rng.normal(size=S).astype(np.float32) for _ in range(N)]
    ar = C.all_reduce(xs, dtype, op, "ring")
    rs = C.reduce_scatter(xs, dtype, dtype, op, "ring")
    ag = C.all_gather(rs)
    for r in range(N):
        assert np.array_equal(ar[r].view(np.uint8), ag[r].view(np.uint8))
        assert np.array_equal(ar[r].view(np.uint8), ar[0].view(np.uint8))


def test_reduce_scatter_bf16_to_fp32_avg_owner_rows():
    N, rc = 4, 6
    rng = np.random.default_rng(5)
    xs = [f32_to_bf16(rng.normal(size=N * rc).astype(np.float32)) for _ in range(N)]
    ys = C.reduce_scatter(xs, "bf16", "fp32", "avg", "ring")
    for j in range(N):
        assert ys[j].dtype == np.float32 and len(ys[j]) == rc
        for k in range(rc):
            acc = None
            for t in range(1, N + 1):
                v = bf16_to_f32(xs[(j + t) % N][j * rc + k:j * rc + k + 1])[0]
                acc = v if acc is None else np.float32(acc + v)
            assert ys[j][k] == np.float32(acc / np.float32(N))


def test_special_cases():
    # N = 1: every collective is a copy; avg divides by one
    x = [np.array([1.5, -2.0, 3.25], np.float32)]
    assert np.array_equal(C.all_reduce(x, "fp32", "avg")[0], x[0])
    assert np.array_equal(C.reduce_scatter(x, "fp32")[0], x[0])
    # S = 0
    assert all(len(o) == 0 for o in C.all_reduce([np.zeros(0, np.float32)] * 3, "fp32"))
    # S < N: empty trailing chunks still give a full result on every rank
    xs = [np.array([i + 1.0, 10.0 * (i + 1)], np.float32) for i in range(5)]
    out = C.all_reduce(xs, "fp32", "sum")
    assert all(np.array_equal(o, np.array([15.0, 150.0], np.float32)) for o in out)
    with pytest.raises(ValueError):
        C.all_reduce([np.zeros(4, np.int32)] * 2, "int32", "avg")
    with pytest.raises(ValueError):
        C.reduce_scatter([np.zeros(5, np.float32)] * 2, "fp32")


def test_nan_inf_propagate():
    xs = [np.array([np.nan, np.inf, np.inf, 1.0], np.float32),
          np.array([1.0, 1.0, -np.inf, 3.4e38], np.float32),
          np.array([1.0, 1.0, 1.0, 3.4e38], np.float32)]
    out = C.all_reduce(xs, "fp32", "sum")[0]
    assert np.isnan(out[0]) and out[1] == np.inf and np.isnan(out[2]) and out[3] == np.inf
