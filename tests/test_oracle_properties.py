"""Property-based pins of the oracle (hypothesis, CPU only): random shapes,
and each property re-derived from the definition on the pages by a different
route than the oracle takes, so that a dropped term, a wrong fold start, an
off-by-one chunk edge or a transposed block fails on shapes no fixed case
names.

- The ring reduce-scatter fold (DTLM §2 "Reduce-Scatter", the N = 4 schedule):
  the oracle emulates the ring step by step; here every element is re-folded
  as a plain left fold in the order the schedule fixes for its chunk,
  (j+1, j+2, ..., N-1, 0, ..., j), with float32 scalars.
- int32 sums wrap like the big-integer sum reduced mod 2^32, in any order.
- All-reduce = all-gather(reduce-scatter) (DTLM §2 "All-Reduce").
- Owner chunks partition [0, S) in rank order with ceil(S/N) elements each
  but the trailing ones; uneven dim-0 shards equal torch.chunk's pieces,
  padded with empty shards (DTLM §4 FSDP2).
- DDP buckets (AIG6 §6.2.4, NXMR §5.1): every tensor exactly once, in
  visiting order; a bucket closes at the first tensor that brings it to the
  cap, never earlier.
- All-to-all(v) (DTLM §2, §8): rows labelled with their (source, destination,
  expert, index) arrive at every destination sorted by (expert, source, index).
- The two-level all-reduce of int32 data equals the flat sum.
- The MoE routing plan (DTLM §8): each route lands on its expert's rank, the
  rows of every receive buffer are a bijection, and inside a (local expert,
  source) block the routes keep their route order.
"""

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import buckets as OB
from oracle import collectives as C
from oracle import hierarchical as H
from oracle import moe as M

SETTINGS = dict(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def _f32(rng, N, S):
    return [rng.normal(size=S).astype(np.float32) * np.float32(rng.choice([1e-3, 1.0, 1e3])) for _ in range(N)]


@settings(**SETTINGS)
@given(N=st.integers(1, 9), S=st.integers(0, 60), seed=st.integers(0, 2**31 - 1))
def test_ring_fold_is_the_schedule_left_fold(N, S, seed):
    rng = np.random.default_rng(seed)
    xs = _f32(rng, N, S)
    got = C.all_reduce(xs, "fp32", "sum", "ring")[0]
    c = -(-S // N) if S else 0
    for e in range(S):
        j = e // c                                   # owner of the chunk holding e
        order = [(j + 1 + k) % N for k in range(N)]  # j+1, ..., N-1, 0, ..., j
        acc = np.float32(xs[order[0]][e])
        for r in order[1:]:
            acc = np.float32(acc + xs[r][e])
        assert got[e].view(np.uint32) == acc.view(np.uint32), (e, j)


@settings(**SETTINGS)
@given(N=st.integers(1, 9), S=st.integers(0, 60), seed=st.integers(0, 2**31 - 1),
       order=st.sampled_from(["ring", "rank"]))
def test_int32_sum_wraps_like_the_big_integer_sum(N, S, seed, order):
    rng = np.random.default_rng(seed)
    xs = [rng.integers(-2**31, 2**31, size=S, dtype=np.int64).astype(np.int32) for _ in range(N)]
    got = C.all_reduce(xs, "int32", "sum", order)[0]
    for e in range(S):
        exact = sum(int(xs[r][e]) for r in range(N))
        wrapped = (exact + 2**31) % 2**32 - 2**31
        assert int(got[e]) == wrapped


@settings(**SETTINGS)
@given(N=st.integers(1, 8), rc=st.integers(0, 12), seed=st.integers(0, 2**31 - 1),
       dtype_op=st.sampled_from([("fp32", "sum"), ("fp32", "avg"), ("bf16", "avg"), ("int32", "sum")]))
def test_all_reduce_is_all_gather_of_reduce_scatter(N, rc, seed, dtype_op):
    dtype, op = dtype_op
    rng = np.random.default_rng(seed)
    S = N * rc
    if dtype == "int32":
        xs = [rng.integers(-1000, 1000, size=S).astype(np.int32) for _ in range(N)]
    else:
        xs = _f32(rng, N, S)
        if dtype == "bf16":
            from oracle.numerics import f32_to_bf16
            xs = [f32_to_bf16(x) for x in xs]
    ar = C.all_reduce(xs, dtype, op, "ring")
    ag = C.all_gather(C.reduce_scatter(xs, dtype, dtype, op, "ring"))
    for r in range(N):
        assert np.array_equal(np.asarray(ar[r]).view(np.uint8), np.asarray(ag[r]).view(np.uint8))


@settings(**SETTINGS)
@given(N=st.integers(1, 70), S=st.integers(0, 5000))
def test_owner_chunks_partition_in_rank_order(N, S):
    chunks = C.owner_chunks(S, N)
    assert len(chunks) == N
    c = -(-S // N) if S else 0
    pos = 0
    for j, (lo, hi) in enumerate(chunks):
        assert lo == pos and lo <= hi                     # contiguous, in rank order
        assert hi - lo == max(0, min(c, S - j * c))       # ceil(S/N) but the trailing ones
        pos = hi
    assert pos == S


@settings(**SETTINGS)
@given(rows=st.integers(0, 300), N=st.integers(1, 70))
def test_uneven_shards_are_torch_chunk(rows, N):
    pieces = [int(p.numel()) for p in torch.chunk(torch.arange(rows), N)] if rows else []
    shards = OB.uneven_dim0_shards(rows, N)
    sizes = [hi - lo for lo, hi in shards]
    assert sizes[:len(pieces)] == pieces and all(s == 0 for s in sizes[len(pieces):])
    assert shards[0][0] == 0 and all(shards[i][1] == shards[i + 1][0] for i in range(N - 1))


@settings(**SETTINGS)
@given(numels=st.lists(st.integers(0, 5000), min_size=0, max_size=40), cap=st.integers(1, 30000),
       es=st.sampled_from([2, 4]), reverse=st.booleans())
def test_bucket_closing_rule(numels, cap, es, reverse):
    buckets = OB.assign_buckets(numels, es, cap, reverse)
    visit = list(range(len(numels)))[::-1] if reverse else list(range(len(numels)))
    assert [t for b in buckets for t in b] == visit           # every tensor once, in visiting order
    for i, b in enumerate(buckets):
        assert b, "empty bucket"
        total = sum(numels[t] for t in b) * es
        before_last = total - numels[b[-1]] * es
        assert before_last < cap                              # not closed earlier
        if i < len(buckets) - 1:
            assert total >= cap                               # closed at the cap
    if buckets:
        last = buckets[-1]
        assert sum(numels[t] for t in last[:-1]) * es < cap


@settings(**SETTINGS)
@given(numels=st.lists(st.integers(1, 5000), min_size=1, max_size=30), k=st.integers(1, 30),
       es=st.sampled_from([2, 4]), reverse=st.booleans())
def test_bucket_closes_exactly_at_the_cap(numels, k, es, reverse):
    """A cap equal to the bytes of the first k visited tensors: the first bucket
    is exactly those k tensors (a bucket closes once its bytes reach the cap)."""
    visit = list(range(len(numels)))[::-1] if reverse else list(range(len(numels)))
    k = min(k, len(numels))
    cap = sum(numels[t] for t in visit[:k]) * es
    buckets = OB.assign_buckets(numels, es, cap, reverse)
    assert buckets[0] == visit[:k]


@settings(**SETTINGS)
@given(N=st.integers(1, 5), E=st.integers(1, 4), seed=st.integers(0, 2**31 - 1))
def test_all_to_all_receive_layout(N, E, seed):
    rng = np.random.default_rng(seed)
    splits = rng.integers(0, 4, size=(N, N, E)).astype(np.int64)
    # row label: (s, d, e, i) packed into 4 int32 elements per row; send layout (d, e, rows)
    sends = []
    for s in range(N):
        rows = [(s, d, e, i) for d in range(N) for e in range(E) for i in range(int(splits[s, d, e]))]
        sends.append(np.array(rows, dtype=np.int32).reshape(-1))
    recv = C.all_to_all(sends, splits, 4)
    for d in range(N):
        got = [tuple(int(v) for v in row) for row in np.asarray(recv[d]).reshape(-1, 4)]
        want = sorted([(s, d, e, i) for s in range(N) for e in range(E) for i in range(int(splits[s, d, e]))],
                      key=lambda t: (t[2], t[0], t[3]))
        assert got == want


@settings(**SETTINGS)
@given(R=st.integers(1, 4), S=st.integers(1, 4), count=st.integers(0, 40), seed=st.integers(0, 2**31 - 1),
       order=st.sampled_from(["ring", "rank"]))
def test_two_level_int32_equals_flat_sum(R, S, count, seed, order):
    rng = np.random.default_rng(seed)
    N = R * S
    xs = [rng.integers(-2**31, 2**31, size=count, dtype=np.int64).astype(np.int32) for _ in range(N)]
    got = H.all_reduce(xs, S, "int32", "sum", order)
    for e in range(count):
        exact = sum(int(xs[r][e]) for r in range(N))
        want = (exact + 2**31) % 2**32 - 2**31
        for r in (0, N - 1):
            assert int(got[r][e]) == want


@settings(**SETTINGS)
@given(N=st.integers(1, 5), E=st.integers(1, 3), K=st.integers(1, 3), seed=st.integers(0, 2**31 - 1))
def test_moe_route_plan_invariants(N, E, K, seed):
    rng = np.random.default_rng(seed)
    G = N * E
    K = min(K, G)
    T = [int(t) for t in rng.integers(0, 12, size=N)]
    experts = []
    for t in T:
        ex = np.array([rng.choice(G, size=K, replace=False) for _ in range(t)], dtype=np.int64).reshape(t, K)
        drop = rng.random(ex.shape) < 0.1
        ex[drop] = -1
        experts.append(ex)
    splits, dest_rank, dest_row = M.route_plan(experts, N, E)
    rows_per_dest = splits.sum(axis=(0, 2))
    seen = [set() for _ in range(N)]
    last = {}
    for s in range(N):
        flat = experts[s].reshape(-1)
        for q, g in enumerate(flat):
            d, r = int(dest_rank[s][q]), int(dest_row[s][q])
            if g < 0:
                assert (d, r) == (-1, -1)
                continue
            assert d == g // E and 0 <= r < rows_per_dest[d]
            assert r not in seen[d]
            seen[d].add(r)
            key = (d, int(g) % E, s)                      # block (local expert, source) on rank d
            assert last.get(key, -1) < r                  # route order kept inside the block
            last[key] = r
    for d in range(N):
        assert seen[d] == set(range(int(rows_per_dest[d])))
    # blocks on rank d: (local expert, source) in that order, each a contiguous run of rows
    spans = {}
    for s in range(N):
        for q, g in enumerate(experts[s].reshape(-1)):
            if g >= 0:
                key = (int(dest_rank[s][q]), int(g) % E, s)
                lo, hi = spans.get(key, (1 << 30, -1))
                spans[key] = (min(lo, int(dest_row[s][q])), max(hi, int(dest_row[s][q])))
    for d in range(N):
        blocks = sorted((e, s) for (dd, e, s) in spans if dd == d)
        run = 0
        for e, s in blocks:
            lo, hi = spans[(d, e, s)]
            assert lo == run and hi - lo + 1 == int(splits[s, d, e])
            run = hi + 1
