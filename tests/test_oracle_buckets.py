"""Pins for the oracle's DDP buckets, FlatParameter layout and uneven shards."""

import numpy as np
import pytest

from gen.workloads import fsdp_layer_tensors, llama7b_tensors
from oracle import buckets as B

MiB = 1 << 20


def test_flat_parameter_worked_example(golden):
    lines = golden("flat_parameter_unit1.txt")
    tensors = [(l[1], int(l[2]), int(l[3]), int(l[4])) for l in lines if l[0] == "tensor"]
    world = int(next(l[1] for l in lines if l[0] == "world"))
    total = int(next(l[1] for l in lines if l[0] == "total"))
    numels = [t[1] for t in tensors]
    intervals, used, padded, shards = B.flat_param_shards(numels, world)
    assert intervals == [(t[2], t[3]) for t in tensors]
    assert used == total and padded == total
    assert shards == [(int(l[2]), int(l[3])) for l in lines if l[0] == "shard"]
    # a tensor may straddle the shard boundary: layer1.bias [6, 8) is split at 7
    name, first, rest = next((l[1], int(l[2]), int(l[3])) for l in lines if l[0] == "split")
    lo, hi = intervals[[t[0] for t in tensors].index(name)]
    assert shards[first][0] <= lo < shards[first][1] and shards[rest][0] < hi <= shards[rest][1]


def test_flat_parameter_padding_to_world_size():
    numels = [6, 2, 4, 2]
    _, used, padded, shards = B.flat_param_shards(numels, 4)
    assert used == 14 and padded == 16 and shards == [(0, 4), (4, 8), (8, 12), (12, 16)]
    flat = B.pack([np.arange(n, dtype=np.uint16) + 1 for n in numels], [0, 1, 2, 3], numels, pad_to=4)
    assert len(flat) == 16 and flat[14] == 0 and flat[15] == 0 and flat[13] == 2


def test_uneven_shards_worked_examples(golden):
    lines = golden("uneven_shards.txt")
    cases, cur = [], None
    for l in lines:
        if l[0] == "case":
            cur = (int(l[1]), int(l[2]), [])
            cases.append(cur)
        else:
            cur[2].append((int(l[2]), int(l[3])))
    for rows, ws, want in cases:
        assert B.uneven_dim0_shards(rows, ws) == want


def test_llama7b_parameter_count_matches_table():
    numels = [n for _, n in llama7b_tensors()]
    assert sum(numels) == 6_738_415_616
    assert round(sum(numels) / 1e6) == 6738           # AIG6 Table 6-5, TP = 1: 6,738 M per GPU


def test_llama7b_buckets():
    names = [n for n, _ in llama7b_tensors()]
    numels = [n for _, n in llama7b_tensors()]
    cap = 25 * MiB
    bks = B.assign_buckets(numels, 2, cap, reverse=True)
    assert len(bks) == 226
    flat = [t for b in bks for t in b]
    assert flat == list(range(len(numels) - 1, -1, -1))       # reverse order, each tensor exactly once
    assert sum(sum(numels[t] for t in b) for b in bks) == sum(numels)
    for b in bks[:-1]:                                          # a bucket closes the moment it reaches the cap
        nbytes = sum(numels[t] for t in b) * 2
        assert nbytes >= cap and nbytes - numels[b[-1]] * 2 < cap
    assert [names[t] for t in bks[0]] == ["lm_head"]
    assert [names[t] for t in bks[1]] == ["final_norm", "layers.31.mlp_norm", "layers.31.attn_norm",
                                          "layers.31.down_proj"]
    assert [names[t] for t in bks[-1]] == ["embed_tokens"]
    sizes = sorted(sum(numels[t] for t in b) for b in bks)
    assert sizes[0] == 16_777_216 and sizes[-1] == 131_072_000
    assert all(s % 8 == 0 for s in sizes)


def test_bucket_rule_small_cases():
    assert B.assign_buckets([10, 10, 10], 1, 15, reverse=False) == [[0, 1], [2]]
    assert B.assign_buckets([10, 10, 10], 1, 15, reverse=True) == [[2, 1], [0]]
    assert B.assign_buckets([10, 10, 10], 1, 10, reverse=False) == [[0], [1], [2]]
    assert B.assign_buckets([5, 100, 5], 1, 50, reverse=False) == [[0, 1], [2]]
    assert B.assign_buckets([], 2, 10) == []
    assert B.assign_buckets([0, 0, 3], 4, 8, reverse=False) == [[0, 1, 2]]


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(0)
    numels = [5, 0, 17, 1, 64, 3]
    tensors = [rng.integers(0, 65535, size=n).astype(np.uint16) for n in numels]
    for cap in (1, 30, 1000):
        for pad in (1, 4, 7):
            for b in B.assign_buckets(numels, 2, cap, reverse=True):
                flat = B.pack(tensors, b, numels, pad_to=pad)
                offs, used, padded = B.bucket_layout(b, numels, pad)
                assert len(flat) == padded and padded % pad == 0 and padded - used < pad
                assert np.all(flat[used:] == 0)
                back = B.unpack(flat, b, numels)
                assert set(back) == set(b)
                for t in b:
                    assert np.array_equal(back[t], tensors[t])


def test_fsdp_layer_flat_size():
    numels = [n for _, n in fsdp_layer_tensors()]
    _, used, padded, shards = B.flat_param_shards(numels, 64)
    assert used == 202_383_360 and padded == used and shards[1] == (3_162_240, 6_324_480)


def test_bucket_all_reduce_is_pack_allreduce_unpack():
    from oracle import collectives as C
    from oracle.numerics import f32_to_bf16
    rng = np.random.default_rng(11)
    N = 3
    numels = [5, 1, 9, 4]
    tensors = [[f32_to_bf16(rng.normal(size=n).astype(np.float32)) for n in numels] for _ in range(N)]
    b = [3, 1, 0]
    out = B.bucket_all_reduce(tensors, b, numels, "bf16", "avg", "ring", pad_to=4)
    # written out by hand: the packed bucket is 4 + 1 + 5 = 10 elements padded to 12, chunks of 4
    flat = [np.concatenate([tensors[r][3], tensors[r][1], tensors[r][0], np.zeros(2, np.uint16)]) for r in range(N)]
    full = C.all_reduce(flat, "bf16", "avg", "ring")
    for r in range(N):
        assert np.array_equal(out[r][3], full[r][0:4])
        assert np.array_equal(out[r][1], full[r][4:5])
        assert np.array_equal(out[r][0], full[r][5:10])
        assert 2 not in out[r]


def test_sum_of_squares_closed_forms():
    from fractions import Fraction
    from oracle.numerics import f32_to_bf16
    assert B.sum_of_squares(np.full(10, 3.0, np.float32), "fp32") == 90
    assert B.sum_of_squares(f32_to_bf16(np.array([0.5, -0.25], np.float32)), "bf16") == Fraction(5, 16)
    assert B.sum_of_squares(np.zeros(0, np.float32), "fp32") == 0
    x = np.random.default_rng(0).normal(size=500).astype(np.float32)
    import math
    assert abs(float(B.sum_of_squares(x, "fp32")) - math.fsum(float(v) ** 2 for v in x)) < 1e-12
