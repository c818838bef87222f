"""The library's calls captured in HIP graphs (torch.cuda.CUDAGraph): no call
allocates, memsets or synchronises, and every launch goes to the caller's
stream, so a captured step replays as recorded.  Each graph is replayed
several times with fresh inputs written eagerly between replays, and every
replay is checked against the oracle."""

import numpy as np
import pytest
import torch

import collective_communication_reduction_amd as gc
from gen import host as G
from gen.workloads import route_tokens
from oracle import buckets as OB
from oracle import collectives as C
from oracle import moe as M
from tests.gpu_util import DEV, assert_same, empty, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _bf16(N, S, seed):
    return [G.normal_bf16(G.stream_key(seed, r, 0), np.arange(S), 1e-3) for r in range(N)]


def _capture(fn):
    """Warm up on a side stream (as torch requires), then capture fn into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_all_reduce_and_reduce_scatter_replayed():
    N, S = 8, 8 * 4096 + 40
    send = [empty(S, "bf16") for _ in range(N)]
    recv = [empty(S, "bf16") for _ in range(N)]
    shards = [empty(S // N, "fp32") for _ in range(N)]

    def step():
        gc.gc_all_reduce(send, recv, op="avg", order="ring")
        gc.gc_reduce_scatter(send, shards, op="avg", order="ring")
    g = _capture(step)
    for rep in range(4):
        xs = _bf16(N, S, seed=100 + rep)
        for t, x in zip(send, xs):
            t.copy_(to_dev(x, "bf16"))
        for t in recv:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = C.all_reduce(xs, "bf16", "avg", "ring")[0]
        for r in (0, N - 1):
            assert_same(from_dev(recv[r]), want, "bf16", f"replay {rep} rank {r}")
        want_rs = C.reduce_scatter(xs, "bf16", "fp32", "avg", "ring")
        for j in range(N):
            assert_same(from_dev(shards[j]), want_rs[j], "fp32", f"replay {rep} owner {j}")


def test_zero_copy_bucket_all_reduce_with_norm_replayed():
    N = 4
    numels = [1000, 37, 4096, 8, 513]
    plan = gc.BucketPlan(numels, "bf16", cap_bytes=6000, reverse=True, pad_to=N)
    try:
        tensors = [[empty(n, "bf16") for n in numels] for _ in range(N)]
        flat = gc.gc_pointers([t for row in tensors for t in row])
        sumsq = torch.zeros(1, dtype=torch.float64, device=DEV)

        def step():
            sumsq.zero_()                       # a fill kernel, recorded in the graph
            for b in range(plan.nbuckets):
                plan.all_reduce(b, flat, N, op="avg", order="ring", sumsq=sumsq)
        g = _capture(step)
        for rep in range(3):
            data = [[G.normal_bf16(G.stream_key(7 + rep, r, t), np.arange(n), 1e-2) for t, n in enumerate(numels)]
                    for r in range(N)]
            for r in range(N):
                for t in range(len(numels)):
                    tensors[r][t].copy_(to_dev(data[r][t], "bf16"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            total = 0.0
            for b in range(plan.nbuckets):
                bucket = plan.bucket_tensors(b)
                want = OB.bucket_all_reduce(data, bucket, numels, "bf16", "avg", "ring", pad_to=N)
                for t in bucket:
                    assert_same(from_dev(tensors[2][t]), want[2][t], "bf16", f"replay {rep} tensor {t}")
                    total += float(OB.sum_of_squares(want[0][t], "bf16"))
            assert abs(float(sumsq.item()) - total) <= 1e-12 * total
    finally:
        plan.close()


def test_moe_route_dispatch_combine_replayed():
    N, E, K, H = 4, 2, 2, 256
    T = [300, 17, 0, 129]
    weights = [torch.empty(max(1, t * K), dtype=torch.float32, device=DEV) for t in T]
    tokens = [empty(max(1, t * H), "bf16") for t in T]
    ex_dev = [torch.empty(max(1, t * K), dtype=torch.int32, device=DEV) for t in T]
    splits = torch.empty(N * N * E, dtype=torch.int64, device=DEV)
    dest = [torch.empty(max(1, t * K * 2), dtype=torch.int32, device=DEV) for t in T]
    scratch = torch.empty(gc.gc_moe_route_scratch_bytes(T, K, E), dtype=torch.uint8, device=DEV)
    cap = sum(T) * K                                  # receive capacity: every route on one rank
    recv = [empty(cap * H, "bf16") for _ in range(N)]
    out = [empty(max(1, t * H), "bf16") for t in T]

    def step():
        gc.gc_moe_route(ex_dev, T, K, E, splits, dest, scratch)
        gc.gc_moe_dispatch(tokens, T, dest, K, H * 2, recv, [cap] * N)
        gc.gc_moe_combine(recv, [cap] * N, dest, weights, T, K, H, "bf16", out)
    for s in range(N):                                # valid routing for the warm-up and capture
        ex_dev[s].zero_()
        if T[s]:
            ex_dev[s].view(T[s], K)[:, 1] = 1
    g = _capture(step)
    rng = np.random.default_rng(5)
    for rep in range(3):
        experts = [route_tokens(20 + rep, s, T[s], N * E, K, 1.1) for s in range(N)]
        toks = [G.normal_bf16(G.stream_key(30 + rep, s, 0), np.arange(T[s] * H), 1.0) for s in range(N)]
        w = [rng.random((T[s], K)).astype(np.float32) for s in range(N)]
        for s in range(N):
            if T[s]:
                ex_dev[s].copy_(torch.from_numpy(experts[s].reshape(-1).astype(np.int32)))
                tokens[s].copy_(to_dev(toks[s], "bf16"))
                weights[s].copy_(torch.from_numpy(w[s].reshape(-1)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = M.combine(M.dispatch(toks, experts, N, E, H), experts, w, N, E, H, "bf16")
        for s in range(N):
            if T[s]:
                assert_same(from_dev(out[s])[:T[s] * H], want[s], "bf16", f"replay {rep} source {s}")


def test_bucket_pack_all_reduce_unpack_and_all_to_all_replayed():
    """The segment copy in a graph: a DDP bucket step (pack with zero padding,
    all-reduce of the bucket, unpack) and an all-to-all(v) with experts."""
    N = 4
    numels = [1000, 37, 4096, 8, 513, 0, 7]
    plan = gc.BucketPlan(numels, "bf16", cap_bytes=6000, reverse=True, pad_to=N)
    try:
        T = len(numels)
        tensors = [[empty(max(1, n), "bf16")[:n] for n in numels] for _ in range(N)]
        flat = [t for row in tensors for t in row]
        bufs = [[empty(plan.bucket_numel[b], "bf16") for _ in range(N)] for b in range(plan.nbuckets)]
        E, rb = 3, 48
        rng = np.random.default_rng(5)
        splits = rng.integers(0, 40, size=(N, N, E)).astype(np.int64)
        send = [torch.empty(max(1, int(splits[s].sum()) * rb), dtype=torch.uint8, device=DEV) for s in range(N)]
        rrows = splits.sum(axis=(0, 2))
        recv = [torch.empty(max(1, int(rrows[d]) * rb), dtype=torch.uint8, device=DEV) for d in range(N)]

        def step():
            for b in range(plan.nbuckets):
                plan.pack(b, flat, bufs[b], N)
                gc.gc_all_reduce(bufs[b], bufs[b], op="avg", order="ring")
                plan.unpack(b, bufs[b], flat, N)
            gc.gc_all_to_all(send, recv, splits, rb)
        for r in range(N):
            for t in tensors[r]:
                t.zero_()
        g = _capture(step)
        for rep in range(3):
            host = [[G.normal_bf16(G.stream_key(300 + rep, r, t), np.arange(n), 1e-2) for t, n in enumerate(numels)]
                    for r in range(N)]
            for r in range(N):
                for t, n in enumerate(numels):
                    if n:
                        tensors[r][t].copy_(to_dev(host[r][t], "bf16"))
            sends = [rng.integers(0, 256, size=int(splits[s].sum()) * rb, dtype=np.uint8) for s in range(N)]
            for s in range(N):
                if sends[s].size:
                    send[s][:sends[s].size].copy_(torch.from_numpy(sends[s]).to(DEV))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for b in range(plan.nbuckets):
                ts = plan.bucket_tensors(b)
                want = OB.bucket_all_reduce(host, ts, numels, "bf16", "avg", "ring", pad_to=N)
                for t in ts:
                    if numels[t]:
                        for r in (0, N - 1):
                            assert_same(from_dev(tensors[r][t]), want[r][t], "bf16", f"replay {rep} tensor {t}")
            want_a2a = C.all_to_all(sends, splits, rb)
            for d in range(N):
                got = recv[d].cpu().numpy()[:len(want_a2a[d])]
                assert np.array_equal(got, want_a2a[d]), f"replay {rep} all-to-all rank {d}"
    finally:
        plan.close()
