"""Pins for the oracle's all-to-all(v): the pages' send/receive pattern, row conservation, inverse."""

import numpy as np
import pytest

from oracle import collectives as C
from oracle import sampled as SM


def test_pattern_of_the_definition():
    # one expert per rank, one row per block, row content = 10*src + dst (the a_{src,dst} labels)
    N = 4
    splits = np.ones((N, N, 1), dtype=np.int64)
    sends = [np.array([10 * s + d for d in range(N)], dtype=np.int32) for s in range(N)]
    recv = C.all_to_all(sends, splits, row_elems=1)
    for d in range(N):
        assert list(recv[d]) == [10 * s + d for s in range(N)]    # rank d gets a_{0,d}, a_{1,d}, ...


def _labelled(splits, row_elems):
    """Send buffers whose rows name (src, dst, expert, k) so every row's destination is checkable."""
    N, _, E = splits.shape
    sends = []
    for s in range(N):
        rows = []
        for d in range(N):
            for e in range(E):
                for k in range(splits[s, d, e]):
                    rows.append([s, d, e, k] + [7] * (row_elems - 4))
        sends.append(np.array(rows, dtype=np.int64).reshape(-1))
    return sends


@pytest.mark.parametrize("N,E,seed", [(2, 1, 0), (3, 2, 1), (4, 3, 2), (8, 8, 3)])
def test_receive_layout_by_expert_then_source(N, E, seed):
    rng = np.random.default_rng(seed)
    splits = rng.integers(0, 4, size=(N, N, E)).astype(np.int64)
    splits[0, N - 1, E - 1] = 0                     # an empty block
    row = 5
    sends = _labelled(splits, row)
    recv = C.all_to_all(sends, splits, row)
    for d in range(N):
        rows = recv[d].reshape(-1, row)
        want = [(s, d, e, k) for e in range(E) for s in range(N) for k in range(splits[s, d, e])]
        assert [tuple(r[:4]) for r in rows] == want
    # rows are conserved: sum over receivers == sum over senders
    assert sum(len(r) for r in recv) == sum(len(s) for s in sends)


def test_inverse_with_transposed_splits_single_expert():
    rng = np.random.default_rng(7)
    N, row = 5, 3
    splits = rng.integers(0, 6, size=(N, N, 1)).astype(np.int64)
    sends = [rng.integers(0, 1000, size=int(splits[s].sum()) * row) for s in range(N)]
    recv = C.all_to_all(sends, splits, row)
    back = C.all_to_all(recv, np.transpose(splits, (1, 0, 2)), row)
    for s in range(N):
        assert np.array_equal(back[s], sends[s])


def test_sampled_source_rows_match_full_permutation():
    rng = np.random.default_rng(9)
    N, E, row = 4, 3, 2
    splits = rng.integers(0, 5, size=(N, N, E)).astype(np.int64)
    sends = [rng.integers(0, 10**6, size=int(splits[s].sum()) * row) for s in range(N)]
    recv = C.all_to_all(sends, splits, row)
    for d in range(N):
        nrows = len(recv[d]) // row
        src, srow = SM.a2a_source_rows(splits, d, np.arange(nrows))
        for k in range(nrows):
            assert np.array_equal(recv[d][k * row:(k + 1) * row], sends[src[k]][srow[k] * row:(srow[k] + 1) * row])


def test_size_mismatch_rejected():
    with pytest.raises(ValueError):
        C.all_to_all([np.zeros(3), np.zeros(2)], np.ones((2, 2, 1), dtype=np.int64), 1)
