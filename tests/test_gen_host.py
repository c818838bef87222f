"""Host side of the input generator: published SplitMix64 outputs, ranges, moments, routing shape."""

import numpy as np

from gen import host as G
from gen import workloads as W


def test_splitmix64_published_sequence():
    # SplitMix64 seeded with 0 outputs mix64(k * golden) for k = 1, 2, 3 (Steele, Lea & Flood 2014;
    # the same sequence is the reference output of Vigna's splitmix64.c)
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    got = [int(G.u64(0, 0, m)) for m in (1, 2, 3)]
    assert got == want


def test_uniform_range_and_exactness():
    key = G.stream_key(0, 3, 0)
    x = G.uniform_f32(key, np.arange(200_000))
    assert x.dtype == np.float32 and x.min() >= -1.0 and x.max() < 1.0
    assert np.all(x * np.float32(2 ** 23) == np.round(x * np.float32(2 ** 23)))     # dyadic, step 2^-23
    assert abs(float(x.mean())) < 0.01 and abs(float(x.var()) - 1 / 3) < 0.01


def test_normal_moments_and_bf16_truncation():
    key = G.stream_key(0, 1, 0)
    f = G.normal_f32(key, np.arange(400_000), 1e-3)
    assert abs(float(f.mean())) < 2e-5 and abs(float(f.std()) - 1e-3) < 2e-5
    assert float(np.abs(f).max()) <= np.sqrt(3.0) * 2 * 1e-3 + 1e-9
    b = G.normal_bf16(key, np.arange(400_000), 1e-3)
    assert np.array_equal(b, (f.view(np.uint32) >> 16).astype(np.uint16))


def test_keys_differ_by_rank_and_stream():
    keys = {G.stream_key(0, r, s) for r in range(8) for s in range(3)}
    assert len(keys) == 24


def test_moe_routing_shape():
    splits, rows = W.moe_send_layout(0, 8, 1024, 64, 2, 1.1)
    assert splits.shape == (8, 8, 8)
    assert all(int(splits[s].sum()) == 2048 for s in range(8))
    assert all(len(r) == 2048 for r in rows)
    # Zipf(1.1) over 64 experts: destination rank 0 (experts 0-7) takes well over half the rows
    frac0 = splits[:, 0, :].sum() / splits.sum()
    assert 0.5 < frac0 < 0.7
    chosen = W.route_tokens(0, 0, 1024, 64, 2, 1.1)
    assert np.all(chosen[:, 0] != chosen[:, 1])


def test_stream_key_accepts_numpy_integers():
    assert G.stream_key(np.int64(0), np.int64(3), np.int32(1)) == G.stream_key(0, 3, 1)
