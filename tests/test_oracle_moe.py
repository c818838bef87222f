"""Pins for the oracle's MoE dispatch / combine (DTLM §8): a worked example,
invariants of the data flow, and exact-arithmetic checks of the combine."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import collectives as C
from oracle import moe as M
from oracle.numerics import bf16_to_f32, f32_to_bf16


def _golden_case(golden):
    lines = golden("moe_route_n2.txt")
    N, E, T, K = 2, 2, 3, 2
    experts = [np.zeros((T, K), dtype=np.int64) for _ in range(N)]
    dest = {}
    for l in lines:
        if l[0] == "route":
            s, t, k, g, d, r = map(int, l[1:])
            experts[s][t, k] = g
            dest[(s, t, k)] = (d, r)
    return lines, N, E, T, K, experts, dest


def test_worked_example_plan(golden):
    lines, N, E, T, K, experts, dest = _golden_case(golden)
    splits, dr, dw = M.route_plan(experts, N, E)
    for (s, t, k), (d, r) in dest.items():
        assert (dr[s][t * K + k], dw[s][t * K + k]) == (d, r)
    want = np.zeros((N, N, E), dtype=np.int64)
    for l in lines:
        if l[0] == "split":
            s, d, e, n = map(int, l[1:])
            want[s, d, e] = n
    assert np.array_equal(splits, want)


def test_worked_example_dispatch(golden):
    lines, N, E, T, K, experts, _ = _golden_case(golden)
    H = 3
    tokens = [np.array([[100 * s + t, -t, 7] for t in range(T)], dtype=np.int32).reshape(-1) for s in range(N)]
    recv = M.dispatch(tokens, experts, N, E, H)
    for l in lines:
        if l[0] == "recv":
            d, r, s, t = map(int, l[1:])
            assert list(recv[d][r * H:(r + 1) * H]) == [100 * s + t, -t, 7]
    assert [len(x) // H for x in recv] == [5, 7]


def _random_routing(rng, N, E, T, K):
    ex = []
    for s in range(N):
        Ts = T[s] if isinstance(T, (list, tuple)) else T
        rows = [rng.choice(N * E, size=K, replace=False) for _ in range(Ts)]
        ex.append(np.array(rows, dtype=np.int64).reshape(Ts, K))
    return ex


@pytest.mark.parametrize("N,E,T,K,seed", [(2, 1, 5, 1, 0), (3, 2, 9, 2, 1), (4, 3, [7, 0, 11, 1], 2, 2),
                                          (8, 8, 40, 2, 3), (4, 2, 13, 4, 4)])
def test_dispatch_invariants(N, E, T, K, seed):
    rng = np.random.default_rng(seed)
    experts = _random_routing(rng, N, E, T, K)
    H = 2
    tokens = [np.array([[s, t] for t in range(len(experts[s]))], dtype=np.int64).reshape(-1) for s in range(N)]
    splits, dr, dw = M.route_plan(experts, N, E)
    recv = M.dispatch(tokens, experts, N, E, H)
    # every copy lands at its planned row on the rank owning its expert, with its token's content
    hit = [np.zeros(len(recv[d]) // H, dtype=np.int64) for d in range(N)]
    for s in range(N):
        Ts = len(experts[s])
        for t in range(Ts):
            for k in range(K):
                g = int(experts[s][t, k])
                d, r = int(dr[s][t * K + k]), int(dw[s][t * K + k])
                assert d == g // E
                assert list(recv[d][r * H:(r + 1) * H]) == [s, t]
                hit[d][r] += 1
    assert all(np.all(h == 1) for h in hit)                 # a bijection onto the receive rows
    assert int(splits.sum()) == sum(len(e) * K for e in experts)
    # inside a destination: blocks by local expert, then source; tokens ascending in a block
    roff = C.a2a_recv_offsets(splits)
    for d in range(N):
        rows = recv[d].reshape(-1, H)
        for e in range(E):
            for s in range(N):
                blk = rows[roff[s, d, e]:roff[s, d, e] + splits[s, d, e]]
                assert np.all(blk[:, 0] == s) and np.all(np.diff(blk[:, 1]) > 0)
                assert all(int(experts[s][t].tolist().count(d * E + e)) == 1 for t in blk[:, 1])


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_combine_top1_unit_weight_is_inverse_of_dispatch(dtype):
    rng = np.random.default_rng(5)
    N, E, T, H = 4, 2, 12, 6
    experts = _random_routing(rng, N, E, T, 1)
    x32 = [rng.normal(size=T * H).astype(np.float32) for _ in range(N)]
    tokens = [f32_to_bf16(x) for x in x32] if dtype == "bf16" else x32
    recv = M.dispatch(tokens, experts, N, E, H)
    out = M.combine(recv, experts, [np.ones((T, 1), np.float32)] * N, N, E, H, dtype)
    for s in range(N):
        assert np.array_equal(out[s], tokens[s])


def test_combine_is_inverse_all_to_all_then_unpermute():
    """Gather by plan == All-to-AllV with transposed splits back to the sources,
    then each token sums its copies from the send order."""
    rng = np.random.default_rng(6)
    N, E, T, K, H = 3, 2, 10, 2, 4
    experts = _random_routing(rng, N, E, T, K)
    splits, _, _ = M.route_plan(experts, N, E)
    y = [rng.normal(size=int(splits[:, d].sum()) * H).astype(np.float32) for d in range(N)]
    w = [rng.random((T, K)).astype(np.float32) for _ in range(N)]
    out = M.combine(y, experts, w, N, E, H, "fp32")
    # a destination holds its rows by (expert, source); the return trip sends them
    # by (source, expert), so reorder the blocks, then plain All-to-AllV with the
    # transposed per-rank splits: source s gets them back in its send order
    roff = C.a2a_recv_offsets(splits)
    ret = []
    for d in range(N):
        rows = y[d].reshape(-1, H)
        ret.append(np.concatenate([rows[roff[s, d, e]:roff[s, d, e] + splits[s, d, e]]
                                   for s in range(N) for e in range(E)]).reshape(-1))
    back = C.all_to_all(ret, np.transpose(splits.sum(axis=2, keepdims=True), (1, 0, 2)), H)
    for s in range(N):
        g = experts[s].reshape(-1)
        tok = np.repeat(np.arange(T), K)
        kk = np.tile(np.arange(K), T)
        order = np.lexsort((tok, g))
        rows = back[s].reshape(-1, H)
        acc = np.zeros((T, H), np.float32)
        first = np.ones(T, bool)
        for k in range(K):
            for pos, i in enumerate(order):
                if kk[i] != k:
                    continue
                t = tok[i]
                p = np.float32(w[s][t, k]) * rows[pos]
                acc[t] = p if first[t] else acc[t] + p
                first[t] = False
        assert np.array_equal(out[s].reshape(T, H), acc)


def _f32(x):
    return float(np.float32(x))


def test_combine_fold_order_and_product_rounding():
    # products and partial sums below are exact in double, so each np.float32() is one rounding
    one, u = 1.0, 2.0 ** -24
    y = np.array([[[one]], [[u]], [[u]]], dtype=np.float32)          # K=3, n=1, H=1
    w = np.ones((1, 3), np.float32)
    got = float(M.combine_rows(y, w, "fp32")[0, 0])
    assert got == _f32(_f32(one + u) + u) == 1.0                      # left fold from k = 0
    assert got != _f32(one + _f32(u + u))
    # each product is rounded to fp32 before it is added (no fused multiply-add)
    a = 1.0 + 2.0 ** -23
    y = np.array([[[a]], [[-(1.0 + 2.0 ** -22)]]], dtype=np.float32)
    w = np.array([[a, 1.0]], dtype=np.float32)
    assert float(M.combine_rows(y, w, "fp32")[0, 0]) == 0.0          # fused: 2^-46


def test_combine_bf16_output_rounds_to_nearest_even():
    ys = f32_to_bf16(np.array([1.0, 2.0 ** -8, 3 * 2.0 ** -8, -2.0 ** -8], np.float32))
    cases = [((0, 1), 1.0), ((0, 2), 1.0 + 2.0 ** -6), ((0, 3), 1.0 - 2.0 ** -8)]
    for (i, j), want in cases:
        y = np.array([[[ys[i]]], [[ys[j]]]], dtype=np.uint16)
        got = M.combine_rows(y, np.ones((1, 2), np.float32), "bf16")
        assert float(bf16_to_f32(got)[0, 0]) == want


def test_combine_closed_form_dyadic():
    rng = np.random.default_rng(8)
    K, n, H = 4, 5, 16
    yv = rng.integers(-64, 65, size=(K, n, H)).astype(np.float32)
    wv = (rng.integers(0, 16, size=(n, K)) / 16.0).astype(np.float32)
    got = M.combine_rows(yv, wv, "fp32")
    for t in range(n):
        for h in range(H):
            exact = sum(Fraction(float(wv[t, k])) * Fraction(float(yv[k, t, h])) for k in range(K))
            assert Fraction(float(got[t, h])) == exact
    # sums of at most 4 * 8 on a grid of 1/2 need 7 significant bits: exact in bf16 as well
    ys = rng.integers(-8, 9, size=(K, n, H)).astype(np.float32)
    ws = (rng.integers(0, 3, size=(n, K)) / 2.0).astype(np.float32)
    got16 = bf16_to_f32(M.combine_rows(f32_to_bf16(ys.reshape(-1)).reshape(K, n, H), ws, "bf16"))
    want = np.einsum("tk,kth->th", ws.astype(np.float64), ys.astype(np.float64))
    assert np.array_equal(got16.astype(np.float64), want)


def test_empty_source_and_no_copies():
    experts = [np.zeros((0, 2), np.int64), np.array([[0, 1]], np.int64)]
    splits, dr, dw = M.route_plan(experts, 2, 1)
    assert splits[0].sum() == 0 and list(splits[1].reshape(-1)) == [1, 1]
    recv = M.dispatch([np.zeros(0, np.float32), np.array([5.0, 6.0], np.float32)], experts, 2, 1, 2)
    assert list(recv[0]) == [5.0, 6.0] and list(recv[1]) == [5.0, 6.0]
    out = M.combine(recv, experts, [np.zeros((0, 2), np.float32), np.array([[0.5, 0.25]], np.float32)],
                    2, 1, 2, "fp32")
    assert len(out[0]) == 0 and list(out[1]) == [3.75, 4.5]


def test_dropped_routes():
    # expert ids outside [0, N*E) are dropped: the plan equals the plan without them
    N, E = 2, 2
    experts = [np.array([[3, -1], [4, 0], [1, 2]], np.int64), np.array([[-5, 7]], np.int64)]
    kept = [np.array([[3], [0], [1]], np.int64), np.zeros((1, 0), np.int64)]
    splits, dr, dw = M.route_plan(experts, N, E)
    ref_splits, _, _ = M.route_plan([np.array([[3], [0], [1], [2]], np.int64), np.zeros((0, 1), np.int64)], N, E)
    assert np.array_equal(splits, ref_splits)
    assert list(dr[0]) == [1, -1, -1, 0, 0, 1] and list(dw[0][[1, 2]]) == [-1, -1]
    assert list(dr[1]) == [-1, -1]
    H = 2
    toks = [np.array([1, 2, 3, 4, 5, 6], np.float32), np.array([7, 8], np.float32)]
    recv = M.dispatch(toks, experts, N, E, H)
    assert sum(len(r) for r in recv) == 4 * H
    w = [np.full((3, 2), 0.5, np.float32), np.ones((1, 2), np.float32)]
    out = M.combine(recv, experts, w, N, E, H, "fp32")
    # token 0 keeps only k = 0; token 1 only k = 1; token 2 both; source 1's token none
    assert list(out[0]) == [0.5, 1.0, 1.5, 2.0, 5.0, 6.0]
    assert list(out[1]) == [0.0, 0.0] and not np.signbit(out[1]).any()
    # a kept -0 product is the fold's start, not 0 + (-0)
    y = np.array([[[0.0]], [[-0.0]]], np.float32)
    got = M.combine_rows(y, np.ones((1, 2), np.float32), "fp32", keep=np.array([[False, True]]))
    assert np.signbit(got[0, 0])
