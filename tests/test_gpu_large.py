"""GPU parity past 2^31 (and 2^32) elements per rank: the sizes where a 32-bit
element or byte index would wrap.  Each call is checked on sampled outputs (random
positions, every chunk edge, and the positions around 2^31 and 2^32 bytes)
that the oracle computes one by one from inputs it regenerates on the host."""

import numpy as np
import pytest
import torch

import collective_communication_reduction_amd as gc
from gen import device as GD
from gen import host as G
from oracle import sampled as SM
from tests.gpu_util import DEV, assert_same, from_dev

pytestmark = pytest.mark.gpu

BIG = (1 << 31) + 9


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _gather(t, pos):
    return from_dev(t.index_select(0, torch.from_numpy(pos.astype(np.int64)).to(DEV)))


def _positions(S, N, rng, extra=()):
    c = -(-S // N)
    pts = [0, 1, S - 2, S - 1, (1 << 31) - 1, 1 << 31, (1 << 31) + 1, (1 << 30) - 1, 1 << 30, (1 << 30) + 1]
    for j in range(N):
        lo, hi = min(S, j * c), min(S, (j + 1) * c)
        pts += [lo, lo + 1, hi - 2, hi - 1]
    pos = np.concatenate([rng.integers(0, S, size=1 << 15), np.array(pts + list(extra), dtype=np.int64)])
    return np.unique(pos[(pos >= 0) & (pos < S)])


def _filled(N, count, dtype, seed, sigma=1e-3):
    keys = [G.stream_key(seed, r, 0) for r in range(N)]
    bufs = []
    for r in range(N):
        if dtype == "bf16":
            t = torch.empty(count, dtype=torch.bfloat16, device=DEV)
            GD.fill_normal_bf16(t, keys[r], sigma)
        else:
            t = torch.empty(count, dtype=torch.float32, device=DEV)
            GD.fill_uniform_f32(t, keys[r])
        bufs.append(t)
    return keys, bufs


def _host_values(keys, pos, dtype, sigma=1e-3):
    if dtype == "bf16":
        return np.stack([G.normal_bf16(k, pos, sigma) for k in keys])
    return np.stack([G.uniform_f32(k, pos.astype(np.uint64)) for k in keys])


@pytest.mark.parametrize("dtype,op", [("bf16", "avg"), ("fp32", "sum")])
def test_all_reduce_past_2_31_elements(dtype, op):
    N, S = 2, BIG
    keys, send = _filled(N, S, dtype, seed=41)
    recv = [torch.empty_like(send[0]) for _ in range(N)]
    gc.gc_all_reduce(send, recv, op=op, order="ring")
    torch.cuda.synchronize()
    pos = _positions(S, N, np.random.default_rng(1))
    want = SM.all_reduce_at(_host_values(keys, pos, dtype), pos, S, dtype, op, "ring")
    for r in range(N):
        assert_same(_gather(recv[r], pos), want, dtype, f"rank {r}")


def test_reduce_scatter_and_all_gather_past_2_31_elements():
    N, rc = 2, (1 << 30) + 3                  # full length 2^31 + 6 per rank
    S = N * rc
    keys, send = _filled(N, S, "bf16", seed=42)
    shards = [torch.empty(rc, dtype=torch.float32, device=DEV) for _ in range(N)]
    gc.gc_reduce_scatter(send, shards, op="avg", order="ring")
    torch.cuda.synchronize()
    pos = _positions(S, N, np.random.default_rng(2))
    vals = _host_values(keys, pos, "bf16")
    want = SM.reduce_scatter_at(vals, pos // rc, pos % rc, rc, "bf16", "fp32", "avg", "ring")
    for j in range(N):
        sel = pos // rc == j
        assert_same(_gather(shards[j], pos[sel] % rc), want[sel], "fp32", f"owner {j}")
    del shards
    # all-gather the bf16 inputs' chunks back: recv[d][E] = send[E // rc][E]
    pieces = [send[j][j * rc:(j + 1) * rc] for j in range(N)]
    full = [torch.empty(S, dtype=torch.bfloat16, device=DEV) for _ in range(N)]
    gc.gc_all_gather(pieces, full)
    torch.cuda.synchronize()
    owner = pos // rc
    want = np.array([vals[o, k] for k, o in enumerate(owner)], dtype=np.uint16)
    for d in range(N):
        assert_same(_gather(full[d], pos), want, "bf16", f"all-gather rank {d}")


def test_all_reduce_and_reduce_scatter_past_2_32_elements():
    """Past 2^32 elements per rank (8 GiB of bf16): a 32-bit element count or vector index would wrap here.
    The fused all-reduce and the bf16 -> fp32 reduce-scatter (whose owner chunks exceed 2^31 elements)."""
    N, S = 2, (1 << 32) + 10
    edges = [(1 << 32) - 1, 1 << 32, (1 << 32) + 1, (1 << 32) + 9]
    keys, send = _filled(N, S, "bf16", seed=43)
    recv = [torch.empty_like(send[0]) for _ in range(N)]
    print(f"all-reduce bf16 avg, {N} ranks x {S} elements", flush=True)
    gc.gc_all_reduce(send, recv, op="avg", order="ring")
    torch.cuda.synchronize()
    pos = _positions(S, N, np.random.default_rng(3), edges)
    vals = _host_values(keys, pos, "bf16")
    want = SM.all_reduce_at(vals, pos, S, "bf16", "avg", "ring")
    for r in range(N):
        assert_same(_gather(recv[r], pos), want, "bf16", f"rank {r}")
    del recv
    torch.cuda.empty_cache()
    rc = S // N                                     # 2^31 + 5 elements per owner
    shards = [torch.empty(rc, dtype=torch.float32, device=DEV) for _ in range(N)]
    print(f"reduce-scatter bf16 -> fp32 avg, {N} ranks x {rc} per owner", flush=True)
    gc.gc_reduce_scatter(send, shards, op="avg", order="ring")
    torch.cuda.synchronize()
    want = SM.reduce_scatter_at(vals, pos // rc, pos % rc, rc, "bf16", "fp32", "avg", "ring")
    for j in range(N):
        sel = pos // rc == j
        assert_same(_gather(shards[j], pos[sel] % rc), want[sel], "fp32", f"owner {j}")


def test_two_level_all_reduce_past_2_31_elements():
    N, Sg, S = 4, 2, BIG
    keys, send = _filled(N, S, "bf16", seed=43)
    recv = [torch.empty_like(send[0]) for _ in range(N)]
    gc.gc_hier_all_reduce(send, recv, Sg, op="avg", order="ring")
    torch.cuda.synchronize()
    R = N // Sg
    c1 = -(-S // Sg)
    edges = []
    for i in range(Sg):
        lo = i * c1
        L = min(S, lo + c1) - lo
        c2 = -(-L // R)
        for h in range(R):
            edges += [lo + min(L, h * c2), lo + min(L, (h + 1) * c2) - 1]
    pos = _positions(S, N, np.random.default_rng(3), extra=edges)
    g0, m0 = SM.hier_fold_starts(pos, S, Sg, R, "ring")
    want = SM.hier_reduce_positions(_host_values(keys, pos, "bf16"), Sg, g0, m0, "bf16", "avg", "bf16")
    for r in (0, N - 1):
        assert_same(_gather(recv[r], pos), want, "bf16", f"rank {r}")


def test_all_to_all_past_4_gib_per_rank():
    """Receive buffers of 4.6 GiB: row offsets times row bytes pass 2^32."""
    N, E, rb = 2, 2, 8192
    splits = np.array([[[150_000, 150_000], [100_000, 1]], [[150_000, 150_000], [3, 100_000]]], dtype=np.int64)
    send_rows = splits.sum(axis=(1, 2))
    send = []
    for s in range(N):
        t = torch.empty(int(send_rows[s]) * rb // 2, dtype=torch.bfloat16, device=DEV)
        GD.fill_normal_bf16(t, G.stream_key(44, s, 0), 1.0)
        send.append(t)
    recv_rows = splits.sum(axis=(0, 2))
    recv = [torch.empty(int(n) * rb // 2, dtype=torch.bfloat16, device=DEV) for n in recv_rows]
    gc.gc_all_to_all(send, recv, splits, rb)
    torch.cuda.synchronize()
    H = rb // 2
    for d in range(N):
        n = int(recv_rows[d])
        rows = np.unique(np.concatenate([np.random.default_rng(d).integers(0, n, size=64), [0, n - 1]]))
        src, srow = SM.a2a_source_rows(splits, d, rows)
        want = np.stack([G.normal_bf16(G.stream_key(44, s, 0), int(r) * H + np.arange(H), 1.0)
                         for s, r in zip(src, srow)])
        got = from_dev(recv[d].view(-1, H).index_select(0, torch.from_numpy(rows).to(DEV)))
        assert np.array_equal(got, want), f"rank {d}"


def test_moe_dispatch_combine_past_4_gib_per_rank():
    """One source of 600,000 tokens x 4096 bf16 routed top-1 to one rank: the
    receive buffer holds 4.6 GiB, and the combine reads it back."""
    from oracle import moe as OM
    N, E, K, H = 2, 1, 1, 4096
    T = [600_000, 0]
    experts = [np.zeros((T[0], 1), np.int64), np.zeros((0, 1), np.int64)]
    ex_dev = [torch.zeros(T[0], dtype=torch.int32, device=DEV), torch.zeros(1, dtype=torch.int32, device=DEV)]
    splits = torch.empty(N * N * E, dtype=torch.int64, device=DEV)
    dest = [torch.empty(T[0] * 2, dtype=torch.int32, device=DEV), torch.empty(2, dtype=torch.int32, device=DEV)]
    scratch = torch.empty(gc.gc_moe_route_scratch_bytes(T, K, E), dtype=torch.uint8, device=DEV)
    gc.gc_moe_route(ex_dev, T, K, E, splits, dest, scratch)
    tok = torch.empty(T[0] * H, dtype=torch.bfloat16, device=DEV)
    GD.fill_normal_bf16(tok, G.stream_key(45, 0, 0), 1.0)
    recv = [torch.empty(T[0] * H, dtype=torch.bfloat16, device=DEV), torch.empty(1, dtype=torch.bfloat16, device=DEV)]
    gc.gc_moe_dispatch([tok, 0], T, dest, K, H * 2, recv, [T[0], 0])
    w = [torch.full((T[0],), 0.5, dtype=torch.float32, device=DEV), torch.ones(1, device=DEV)]
    out = [torch.empty(T[0] * H, dtype=torch.bfloat16, device=DEV), 0]
    gc.gc_moe_combine(recv, [T[0], 0], dest, w, T, K, H, "bf16", out)
    torch.cuda.synchronize()
    _, dr, dw = OM.route_plan(experts, N, E)
    assert np.array_equal(dest[0].cpu().numpy().reshape(-1, 2)[:, 1], dw[0])
    rows = np.unique(np.concatenate([np.random.default_rng(5).integers(0, T[0], size=64), [0, T[0] - 1,
                                                                                          (1 << 31) // (H * 2)]]))
    want = np.stack([G.normal_bf16(G.stream_key(45, 0, 0), int(t) * H + np.arange(H), 1.0) for t in rows])
    got = from_dev(recv[0].view(-1, H).index_select(0, torch.from_numpy(dw[0][rows]).to(DEV)))
    assert np.array_equal(got, want)
    comb = OM.combine_rows(want[None], np.full((len(rows), 1), 0.5, np.float32), "bf16")
    assert_same(from_dev(out[0].view(-1, H).index_select(0, torch.from_numpy(rows).to(DEV))).reshape(-1),
                comb.reshape(-1), "bf16", "combine")
