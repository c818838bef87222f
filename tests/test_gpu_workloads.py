"""GPU parity at the five workloads' full sizes, in the launch configuration and
HBM layout bench.py times (a RankArena: each rank's buffers in its own region
of HBM, the workload's stagger between ranks: 4 KiB, 64 KiB for 16 ranks).

At these sizes the step-by-step oracle cannot hold the inputs at once.  The
reductions of the all-reduce, FSDP, two-level and HSDP workloads are still
compared with the oracle element by element: the inputs of one owner chunk
(one cell of the two-level schedule) at a time are copied back from the
device generator's buffers (its bits are pinned to the host generator's) and
folded by the oracle's whole-chunk evaluators, which are themselves pinned to
the step-by-step emulation.  The DDP and MoE workloads check sampled outputs
the oracle computes one by one from inputs it regenerates on the host by index
(random positions plus every chunk edge).  Properties that hold at any size are
checked on the device as well: every rank's result is identical, fused ==
reduce-scatter + all-gather bit for bit, and data movement equals the
permutation the oracle derives.  The 4-rank fp32 all-reduce is small enough for
a full step-by-step oracle comparison."""

import os

import numpy as np
import pytest
import torch

import collective_communication_reduction_amd as gc
from gen import device as GD
from gen import host as G
from gen.workloads import WORKLOADS, fsdp_layer_tensors, llama7b_tensors, moe_send_layout
from oracle import buckets as OB
from oracle import collectives as C
from oracle import sampled as SM
from tests.gpu_util import DEV, assert_same, from_dev, max_ulp

pytestmark = pytest.mark.gpu

SEED = 0


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _positions(S, N, rng, m=1 << 18):
    """Random positions plus the first and last two elements of every owner chunk."""
    c = -(-S // N)
    edges = []
    for j in range(N):
        lo, hi = min(S, j * c), min(S, (j + 1) * c)
        edges += [lo, lo + 1, hi - 2, hi - 1]
    pos = np.concatenate([rng.integers(0, S, size=m), np.array(edges)])
    pos = pos[(pos >= 0) & (pos < S)]
    return np.unique(pos)


def _gather(t, pos):
    idx = torch.from_numpy(pos.astype(np.int64)).to(DEV)
    return from_dev(t.index_select(0, idx))


def _slices(bufs, lo, hi):
    """Host copy of elements [lo, hi) of every rank's buffer, one row per rank."""
    return list(from_dev(torch.stack([b[lo:hi] for b in bufs])))


def test_ar_fp32_n4_full():
    cfg = WORKLOADS["ar_fp32_n4"]
    N, S = cfg["nranks"], cfg["count"]
    xs = [G.uniform_f32(G.stream_key(SEED, r, 0), np.arange(S)) for r in range(N)]
    want = C.all_reduce(xs, "fp32", "sum", "ring")[0]
    arena = gc.RankArena(N)
    send = arena.alloc(S, "fp32")
    for r in range(N):
        GD.fill_uniform_f32(send[r], G.stream_key(SEED, r, 0))
    for algo in ("fused", "rs_ag"):
        recv = arena.alloc(S, "fp32")
        scratch = torch.empty(gc.gc_all_reduce_scratch_bytes(S, N, "fp32"), dtype=torch.uint8, device=DEV)
        gc.gc_all_reduce(send, recv, op="sum", order="ring", algo=algo, scratch=scratch)
        torch.cuda.synchronize()
        for r in range(N):
            assert_same(from_dev(recv[r]), want, "fp32", f"{algo} rank {r}")


def test_ar_bf16_n8_full():
    cfg = WORKLOADS["ar_bf16_n8"]
    N, S, sigma = cfg["nranks"], cfg["count"], cfg["sigma"]
    arena = gc.RankArena(N)
    send = arena.alloc(S, "bf16")
    keys = [G.stream_key(SEED, r, 0) for r in range(N)]
    for r in range(N):
        GD.fill_normal_bf16(send[r], keys[r], sigma)
    recv = arena.alloc(S, "bf16")
    gc.gc_all_reduce(send, recv, op="avg", order="ring", algo="fused")
    # the same all-reduce as reduce-scatter then all-gather, separately
    recv2 = arena.alloc(S, "bf16")
    scratch = torch.empty(gc.gc_all_reduce_scratch_bytes(S, N, "bf16"), dtype=torch.uint8, device=DEV)
    gc.gc_all_reduce(send, recv2, op="avg", order="ring", algo="rs_ag", scratch=scratch)
    torch.cuda.synchronize()
    for r in range(N):
        assert torch.equal(recv[r].view(torch.int16), recv[0].view(torch.int16)), f"rank {r} differs"
        assert torch.equal(recv2[r].view(torch.int16), recv[0].view(torch.int16)), f"rs_ag rank {r} differs"
    # every output, owner chunk by owner chunk (rank 3's copy; all ranks are equal above)
    c = -(-S // N)
    for j in range(N):
        lo, hi = min(S, j * c), min(S, (j + 1) * c)
        want = SM.reduce_scatter_owner(_slices(send, lo, hi), j, "bf16", "bf16", "avg", "ring")
        got = from_dev(recv[3][lo:hi])
        assert max_ulp(got, want) <= 1
        assert_same(got, want, "bf16", f"chunk {j}")
    # and sampled positions against inputs the oracle regenerates on the host
    pos = _positions(S, N, np.random.default_rng(1), m=1 << 14)
    vals = np.stack([G.normal_bf16(keys[r], pos, sigma) for r in range(N)])
    assert_same(_gather(recv[3], pos), SM.all_reduce_at(vals, pos, S, "bf16", "avg", "ring"), "bf16", "sampled")


def _llama_layout():
    numels = [n for _, n in llama7b_tensors()]
    offs = np.concatenate([[0], np.cumsum(numels)]).astype(np.int64)
    return numels, offs


# one bucket of every composition the 226-bucket plan has: lm_head alone; final norm + layer 31's norms and
# down_proj; then a layer's up, gate, o, v, k, q and [norms, down_proj] (each repeated 31-32 times); embedding
FULL_BUCKETS = (0, 1, 2, 3, 4, 5, 6, 7, 8, 225)


def _full_buckets(nbuckets):
    """The buckets compared in full: all of them (every output of the step, about 80 s of host-side
    folding per step on the GPU machine), or with GC_DDP_ALL_BUCKETS=0 one bucket of each composition."""
    if os.environ.get("GC_DDP_ALL_BUCKETS", "1") in ("", "0"):
        return FULL_BUCKETS
    return range(nbuckets)


def _ddp_bucket_full(result, b, ts, numels, offs, keys, sigma, N):
    """Every output of bucket b against the oracle's all-reduce of the packed bucket.  The inputs (consumed
    in place by the step) are regenerated by index with the device generator, which is pinned bit for bit to
    the host one, and packed on the host in the bucket's order."""
    boffs, used, _ = OB.bucket_layout(ts, numels)
    tmp = torch.empty(max(numels[t] for t in ts), dtype=torch.bfloat16, device=DEV)
    packed = np.empty((N, used), dtype=np.uint16)
    for r in range(N):
        for t, o in zip(ts, boffs):
            GD.fill_normal_bf16(tmp[:numels[t]], keys[r], sigma, base=int(offs[t]))
            packed[r, o:o + numels[t]] = from_dev(tmp[:numels[t]])
    got = np.empty(used, dtype=np.uint16)
    for t, o in zip(ts, boffs):
        got[o:o + numels[t]] = from_dev(result[t])
    c = -(-used // N)
    for j in range(N):
        lo, hi = min(used, j * c), min(used, (j + 1) * c)
        if lo < hi:
            want = SM.reduce_scatter_owner([packed[r, lo:hi] for r in range(N)], j, "bf16", "bf16", "avg", "ring")
            assert_same(got[lo:hi], want, "bf16", f"bucket {b} owner chunk {j}")
    print(f"bucket {b}: all {used} outputs equal the oracle", flush=True)


def test_ddp_llama7b_full_step():
    cfg = WORKLOADS["ddp_llama7b"]
    N, sigma, cap = cfg["nranks"], cfg["sigma"], cfg["cap_bytes"]
    numels, offs = _llama_layout()
    total = int(offs[-1])
    keys = [G.stream_key(SEED, r, 0) for r in range(N)]
    arena = gc.RankArena(N, min_bytes=total * 2 + (1 << 30))
    flat = arena.alloc(total, "bf16")
    for r in range(N):
        GD.fill_normal_bf16(flat[r], keys[r], sigma)
    tensors = [flat[r][int(offs[t]):int(offs[t]) + numels[t]] for r in range(N) for t in range(len(numels))]
    plan = gc.BucketPlan(numels, "bf16", cap, reverse=True)
    bufs = [arena.alloc(max(plan.bucket_numel), "bf16") for _ in range(2)]
    for b in range(plan.nbuckets):                      # one step, exactly as bench.py runs it
        views = [x[:plan.bucket_numel[b]] for x in bufs[b & 1]]
        plan.pack(b, tensors, views, N)
        gc.gc_all_reduce(views, views, op="avg", order="ring", algo="fused")
        plan.unpack(b, views, tensors, N)
    torch.cuda.synchronize()
    for r in range(1, N):
        assert torch.equal(flat[r].view(torch.int16), flat[0].view(torch.int16)), f"rank {r} differs"
    # sampled outputs of every bucket: bucket element e -> (tensor, index) -> model-order flat index
    rng = np.random.default_rng(2)
    oracle_buckets = OB.assign_buckets(numels, 2, cap, reverse=True)
    assert plan.nbuckets == len(oracle_buckets)
    flat_pos, want = [], []
    for b, ts in enumerate(oracle_buckets):
        boffs, used, _ = OB.bucket_layout(ts, numels)
        e = np.unique(np.concatenate([rng.integers(0, used, size=48), [0, used - 1],
                                      [min(used - 1, j * -(-used // N)) for j in range(N)]]))
        starts = np.asarray(boffs)
        which = np.searchsorted(starts, e, side="right") - 1
        fidx = np.array([offs[ts[w]] + (ee - starts[w]) for w, ee in zip(which, e)], dtype=np.int64)
        vals = np.stack([G.normal_bf16(keys[r], fidx, sigma) for r in range(N)])
        want.append(SM.all_reduce_at(vals, e, used, "bf16", "avg", "ring"))
        flat_pos.append(fidx)
    flat_pos = np.concatenate(flat_pos)
    want = np.concatenate(want)
    got = _gather(flat[5], flat_pos)
    assert max_ulp(got, want) <= 1
    assert_same(got, want, "bf16", "sampled bucket outputs")
    T = len(numels)
    for b in _full_buckets(plan.nbuckets):              # every output of every bucket
        _ddp_bucket_full(tensors[5 * T:6 * T], b, oracle_buckets[b], numels, offs, keys, sigma, N)
    plan.close()


def test_ddp_llama7b_zero_copy_full_step():
    # the bench's zero-copy step: every bucket all-reduced in place over the gradient tensors,
    # with the sum of squares of the synced gradients accumulated on the device
    cfg = WORKLOADS["ddp_llama7b"]
    N, sigma, cap = cfg["nranks"], cfg["sigma"], cfg["cap_bytes"]
    numels, offs = _llama_layout()
    total = int(offs[-1])
    keys = [G.stream_key(SEED, r, 0) for r in range(N)]
    arena = gc.RankArena(N, min_bytes=total * 2 + (1 << 30))
    flat = arena.alloc(total, "bf16")
    for r in range(N):
        GD.fill_normal_bf16(flat[r], keys[r], sigma)
    tensors = [flat[r][int(offs[t]):int(offs[t]) + numels[t]] for r in range(N) for t in range(len(numels))]
    plan = gc.BucketPlan(numels, "bf16", cap, reverse=True)
    sq = torch.zeros(1, dtype=torch.float64, device=DEV)
    for b in range(plan.nbuckets):
        plan.all_reduce(b, tensors, N, op="avg", order="ring", sumsq=sq)
    torch.cuda.synchronize()
    for r in range(1, N):
        assert torch.equal(flat[r].view(torch.int16), flat[0].view(torch.int16)), f"rank {r} differs"
    rng = np.random.default_rng(6)
    oracle_buckets = OB.assign_buckets(numels, 2, cap, reverse=True)
    flat_pos, want = [], []
    for b, ts in enumerate(oracle_buckets):
        boffs, used, _ = OB.bucket_layout(ts, numels)
        e = np.unique(np.concatenate([rng.integers(0, used, size=48), [0, used - 1],
                                      [min(used - 1, j * -(-used // N)) for j in range(N)]]))
        starts = np.asarray(boffs)
        which = np.searchsorted(starts, e, side="right") - 1
        fidx = np.array([offs[ts[w]] + (ee - starts[w]) for w, ee in zip(which, e)], dtype=np.int64)
        vals = np.stack([G.normal_bf16(keys[r], fidx, sigma) for r in range(N)])
        want.append(SM.all_reduce_at(vals, e, used, "bf16", "avg", "ring"))
        flat_pos.append(fidx)
    got = _gather(flat[2], np.concatenate(flat_pos))
    assert_same(got, np.concatenate(want), "bf16", "sampled zero-copy outputs")
    T = len(numels)
    for b in _full_buckets(plan.nbuckets):              # every output of every bucket
        _ddp_bucket_full(tensors[2 * T:3 * T], b, oracle_buckets[b], numels, offs, keys, sigma, N)
    # the accumulated sum of squares equals the squared norm of the synced gradients (any order: fp64
    # relative bound over 6.7e9 terms)
    norm2 = 0.0
    for lo in range(0, total, 1 << 28):                     # in pieces: the float64 copy would be 54 GB
        norm2 += float((flat[0][lo:lo + (1 << 28)].double() ** 2).sum().item())
    assert abs(float(sq.item()) - norm2) <= 1e-9 * norm2
    plan.close()


def test_fsdp_layer_n64_full():
    N = WORKLOADS["fsdp_layer_n64"]["nranks"]
    numels = [n for _, n in fsdp_layer_tensors()]
    _, used, S, _ = OB.flat_param_shards(numels, N)
    rc = S // N
    gkeys = [G.stream_key(SEED, r, 0) for r in range(N)]
    pkeys = [G.stream_key(SEED, r, 1) for r in range(N)]
    arena = gc.RankArena(N)
    grads = arena.alloc(S, "bf16")
    for r in range(N):
        GD.fill_normal_bf16(grads[r], gkeys[r], 1e-3)
    gshards = arena.alloc(rc, "fp32")
    gc.gc_reduce_scatter(grads, gshards, op="avg", order="ring")
    torch.cuda.synchronize()
    # all 64 x 3,162,240 fp32 outputs, streamed owner by owner through the oracle
    for j in range(N):
        want = SM.reduce_scatter_owner(_slices(grads, j * rc, (j + 1) * rc), j, "bf16", "fp32", "avg", "ring")
        assert_same(from_dev(gshards[j]), want, "fp32", f"reduce-scatter owner {j}")
    rng = np.random.default_rng(3)
    for j in (0, 29, N - 1):                            # a sample against host-regenerated inputs too
        k = np.unique(np.concatenate([rng.integers(0, rc, size=512), [0, 1, rc - 2, rc - 1]]))
        vals = np.stack([G.normal_bf16(gkeys[i], j * rc + k, 1e-3) for i in range(N)])
        want = SM.reduce_scatter_at(vals, np.full(len(k), j), k, rc, "bf16", "fp32", "avg", "ring")
        assert_same(_gather(gshards[j], k), want, "fp32", f"reduce-scatter owner {j}")
    pshards = arena.alloc(rc, "bf16")
    for r in range(N):
        GD.fill_normal_bf16(pshards[r], pkeys[r], 0.02)
    params = arena.alloc(S, "bf16")
    gc.gc_all_gather(pshards, params)
    torch.cuda.synchronize()
    for d in range(1, N):
        assert torch.equal(params[d].view(torch.int16), params[0].view(torch.int16)), f"rank {d} differs"
    # every output: the all-gather's result is the concatenation of the shards in rank order
    for j in range(N):
        assert torch.equal(params[0][j * rc:(j + 1) * rc].view(torch.int16), pshards[j].view(torch.int16)), j
    pos = _positions(S, N, np.random.default_rng(4), m=1 << 16)
    owner, k = pos // rc, pos % rc
    want = np.array([G.normal_bf16(pkeys[i], np.array([kk]), 0.02)[0] for i, kk in zip(owner, k)], dtype=np.uint16)
    assert_same(_gather(params[17], pos), want, "bf16", "all-gather sampled")


def test_moe_a2a_n8_full():
    cfg = WORKLOADS["moe_a2a_n8"]
    N, H = cfg["nranks"], cfg["hidden"]
    splits, rows = moe_send_layout(SEED, N, cfg["tokens"], cfg["experts"], cfg["topk"], cfg["zipf_s"])
    recv_rows = splits.sum(axis=(0, 2))
    arena = gc.RankArena(N)
    send_full = arena.alloc(max(len(r) for r in rows) * H, "bf16")
    recv_full = arena.alloc(int(recv_rows.max()) * H, "bf16")
    send = [send_full[s][:len(rows[s]) * H] for s in range(N)]
    recv = [recv_full[d][:int(recv_rows[d]) * H] for d in range(N)]
    for s in range(N):
        GD.fill_normal_bf16_rows(send[s], torch.from_numpy(rows[s]).to(DEV), H, G.stream_key(SEED, s, 0), 1.0)
    gc.gc_all_to_all(send, recv, splits, H * 2)
    torch.cuda.synchronize()
    # the oracle's permutation applied to global row ids gives every received row's source row
    base = np.concatenate([[0], np.cumsum([len(r) for r in rows])])
    ids = [np.arange(base[s], base[s + 1], dtype=np.int64) for s in range(N)]
    src_of = C.all_to_all(ids, splits, 1)
    all_send = torch.cat(send).view(-1, H)
    for d in range(N):
        want = all_send.index_select(0, torch.from_numpy(src_of[d]).to(DEV))
        assert torch.equal(recv[d].view(-1, H).view(torch.int16), want.view(torch.int16)), f"rank {d}"
    # sampled rows against values the oracle regenerates from the routing alone
    rng = np.random.default_rng(5)
    for d in (0, 3, 7):
        n = int(recv_rows[d])
        pick = np.unique(np.concatenate([rng.integers(0, n, size=64), [0, n - 1]]))
        srcs, srow = SM.a2a_source_rows(splits, d, pick)
        want = np.stack([G.normal_bf16(G.stream_key(SEED, s, 0), int(rows[s][r]) * H + np.arange(H), 1.0)
                         for s, r in zip(srcs, srow)])
        got = from_dev(recv[d].view(-1, H).index_select(0, torch.from_numpy(pick).to(DEV)))
        assert np.array_equal(got, want), f"rank {d} sampled rows"
    # the skew the workload is meant to have: most rows land on rank 0
    assert 0.55 < recv_rows[0] / recv_rows.sum() < 0.67


def test_moe_ep_n8_full():
    """Routing plan, dispatch and combine at full size, in bench.py's layout.
    The plan is compared with the oracle's for all 262,144 routes; dispatched
    and combined rows are sampled against values the oracle computes from the
    host generator (identity experts: a token's K expert rows are its own row),
    then every dispatched row against the token row its route names and every
    combined row against the oracle's weighted sum of the token's rows."""
    from gen.workloads import route_tokens
    from oracle import moe as OM
    cfg = WORKLOADS["moe_ep_n8"]
    N, T, H, K = cfg["nranks"], cfg["tokens"], cfg["hidden"], cfg["topk"]
    E = cfg["experts"] // N
    experts = [route_tokens(SEED, s, T, cfg["experts"], K, cfg["zipf_s"]) for s in range(N)]
    want_splits, dr, dw = OM.route_plan(experts, N, E)
    arena = gc.RankArena(N)
    tokens = arena.alloc(T * H, "bf16")
    for s in range(N):
        GD.fill_normal_bf16(tokens[s], G.stream_key(SEED, s, 0), 1.0)
    weights = [torch.empty(T * K, dtype=torch.float32, device=DEV) for _ in range(N)]
    for s in range(N):
        GD.fill_uniform_f32(weights[s], G.stream_key(SEED, s, 3))
    ex_dev = [torch.from_numpy(e.reshape(-1).astype(np.int32)).to(DEV) for e in experts]
    splits = torch.empty(N * N * E, dtype=torch.int64, device=DEV)
    dest = [torch.empty(T * K * 2, dtype=torch.int32, device=DEV) for _ in range(N)]
    scratch = torch.empty(gc.gc_moe_route_scratch_bytes([T] * N, K, E), dtype=torch.uint8, device=DEV)
    gc.gc_moe_route(ex_dev, [T] * N, K, E, splits, dest, scratch)
    torch.cuda.synchronize()
    assert np.array_equal(splits.cpu().numpy().reshape(N, N, E), want_splits)
    for s in range(N):
        got = dest[s].cpu().numpy().reshape(-1, 2)
        assert np.array_equal(got[:, 0], dr[s]) and np.array_equal(got[:, 1], dw[s]), f"source {s}"
    rows = [int(x) for x in want_splits.sum(axis=(0, 2))]
    recv_full = arena.alloc(max(rows) * H, "bf16")
    recv = [recv_full[d][:rows[d] * H] for d in range(N)]
    for r in recv:
        r.view(torch.int16).fill_(-1)                      # 0xFFFF, a NaN pattern no token row holds whole
    gc.gc_moe_dispatch(tokens, [T] * N, dest, K, H * 2, recv, rows)
    out = arena.alloc(T * H, "bf16")
    gc.gc_moe_combine(recv, rows, dest, weights, [T] * N, K, H, "bf16", out)
    torch.cuda.synchronize()
    for d in range(N):                                  # every receive row was written
        unwritten = (recv[d].view(-1, H).view(torch.int16) == -1).all(dim=1).sum().item()
        assert unwritten == 0, f"rank {d}: {unwritten} rows not written"
    rng = np.random.default_rng(11)
    for s in (0, 5, 7):
        pick = np.unique(np.concatenate([rng.integers(0, T, size=96), [0, T - 1]]))
        tok_rows = np.stack([G.normal_bf16(G.stream_key(SEED, s, 0), int(t) * H + np.arange(H), 1.0) for t in pick])
        for k in range(K):                              # dispatched copies
            d, r = dr[s][pick * K + k], dw[s][pick * K + k]
            got = np.stack([from_dev(recv[int(dd)].view(-1, H)[int(rr)]) for dd, rr in zip(d, r)])
            assert np.array_equal(got, tok_rows), f"source {s} k {k}"
        w = G.uniform_f32(G.stream_key(SEED, s, 3), np.arange(T * K, dtype=np.uint64)).reshape(T, K)[pick]
        want = OM.combine_rows(np.stack([tok_rows] * K), w, "bf16")
        got = from_dev(out[s].view(-1, H).index_select(0, torch.from_numpy(pick).to(DEV)))
        assert_same(got.reshape(-1), want.reshape(-1), "bf16", f"source {s} combine")
    # every dispatched row is the token row its route names (pure movement, compared on the device) ...
    all_tok = torch.cat([t.view(-1, H) for t in tokens])
    for d in range(N):
        idx = np.full(rows[d], -1, dtype=np.int64)
        for s in range(N):
            m = dr[s] == d
            idx[dw[s][m]] = s * T + np.arange(T * K)[m] // K
        assert (idx >= 0).all()
        want = all_tok.index_select(0, torch.from_numpy(idx).to(DEV))
        assert torch.equal(recv[d].view(-1, H).view(torch.int16), want.view(torch.int16)), f"dispatch rank {d}"
    del all_tok
    # ... and every combined row equals the oracle's weighted sum (identity experts: a token's K rows are its own)
    for s in range(N):
        tok = from_dev(tokens[s]).reshape(T, H)
        w = G.uniform_f32(G.stream_key(SEED, s, 3), np.arange(T * K, dtype=np.uint64)).reshape(T, K)
        want = OM.combine_rows(np.stack([tok] * K), w, "bf16")
        assert_same(from_dev(out[s]).reshape(-1), want.reshape(-1), "bf16", f"source {s} combine, every row")


def _fsdp2_layout(N):
    """Per-parameter shapes, offsets in a rank's flat buffer, and each rank's shard offsets."""
    from gen.workloads import fsdp_layer_shapes
    from oracle import fsdp2 as F2
    shapes = fsdp_layer_shapes()
    rows = [r for _, r, _ in shapes]
    cols = [c for _, _, c in shapes]
    offs = np.concatenate([[0], np.cumsum([r * c for r, c in zip(rows, cols)])]).astype(np.int64)
    sh = [[F2.shard_elems(rows[p], cols[p], N)[r] for p in range(len(rows))] for r in range(N)]
    soffs = [np.concatenate([[0], np.cumsum([hi - lo for lo, hi in sh[r]])]).astype(np.int64) for r in range(N)]
    return rows, cols, offs, sh, soffs


@pytest.mark.parametrize("N", [64, 48])
def test_fsdp2_layer_full(N):
    """FSDP2 per-parameter reduce-scatter (avg, bf16 -> fp32) and all-gather of
    one transformer layer at full size, 64 ranks (every dim divides) and 48
    ranks (uneven shards: 4096 / 48 and 11008 / 48 leave short last shards):
    sampled outputs against host-regenerated inputs, then every output of both
    collectives."""
    rows, cols, offs, sh, soffs = _fsdp2_layout(N)
    P, S = len(rows), int(offs[-1])
    arena = gc.RankArena(N)
    grads = arena.alloc(S, "bf16")
    gkeys = [G.stream_key(SEED, r, 0) for r in range(N)]
    pkeys = [G.stream_key(SEED, r, 1) for r in range(N)]
    for r in range(N):
        GD.fill_normal_bf16(grads[r], gkeys[r], 1e-3)
    most = max(int(s[-1]) for s in soffs)
    gsh = arena.alloc(most, "fp32")
    gviews = [[grads[r][offs[p]:offs[p + 1]] for p in range(P)] for r in range(N)]
    sviews = [[gsh[r][soffs[r][p]:soffs[r][p + 1]] if soffs[r][p + 1] > soffs[r][p] else 0 for p in range(P)]
              for r in range(N)]
    gc.gc_fsdp2_reduce_scatter(gviews, sviews, rows, cols, N, "bf16", "fp32", "avg", "ring")
    torch.cuda.synchronize()
    rng = np.random.default_rng(N)
    for p in range(P):
        for j in sorted({0, 1, N // 2, N - 1}):
            lo, hi = sh[j][p]
            n = hi - lo
            if n == 0:
                continue
            k = np.unique(np.concatenate([rng.integers(0, n, size=512), [0, n - 1]]))
            vals = np.stack([G.normal_bf16(gkeys[i], offs[p] + lo + k, 1e-3) for i in range(N)])
            want = SM.reduce_positions(vals, "bf16", np.full(len(k), (j + 1) % N), "avg", "fp32")
            assert_same(_gather(sviews[j][p], k), want, "fp32", f"param {p} owner {j}")
    # every output of every parameter, owner by owner (shard j of parameter p is elements [lo, hi) of p on
    # every rank, folded from rank j + 1; uneven at 48 ranks)
    for p in range(P):
        for j in range(N):
            lo, hi = sh[j][p]
            if hi == lo:
                continue
            a, b = int(offs[p]) + lo, int(offs[p]) + hi
            want = SM.reduce_scatter_owner(_slices(grads, a, b), j, "bf16", "fp32", "avg", "ring")
            assert_same(from_dev(sviews[j][p]), want, "fp32", f"param {p} owner {j}, every output")
    del grads, gsh, gviews, sviews
    psh = arena.alloc(most, "bf16")
    for r in range(N):
        GD.fill_normal_bf16(psh[r], pkeys[r], 0.02)
    params = arena.alloc(S, "bf16")
    pviews = [[params[r][offs[p]:offs[p + 1]] for p in range(P)] for r in range(N)]
    shviews = [[psh[r][soffs[r][p]:soffs[r][p + 1]] if soffs[r][p + 1] > soffs[r][p] else 0 for p in range(P)]
               for r in range(N)]
    gc.gc_fsdp2_all_gather(shviews, pviews, rows, cols, N, "bf16")
    torch.cuda.synchronize()
    for d in range(1, N):
        assert torch.equal(params[d].view(torch.int16), params[0].view(torch.int16)), f"rank {d} differs"
    for p in range(P):                                  # every output: parameter p is its shards in rank order
        parts = [shviews[r][p] for r in range(N) if not isinstance(shviews[r][p], int)]
        assert torch.equal(pviews[0][p].view(torch.int16), torch.cat(parts).view(torch.int16)), f"param {p}"
    for p in range(P):
        n = rows[p] * cols[p]
        e = np.unique(np.concatenate([rng.integers(0, n, size=4096), [0, n - 1]]))
        c_rows = -(-rows[p] // N)
        owner = (e // cols[p]) // c_rows
        local = e - np.array([sh[o][p][0] for o in owner])
        want = np.array([G.normal_bf16(pkeys[o], np.array([soffs[o][p] + l]), 0.02)[0] for o, l in zip(owner, local)],
                        dtype=np.uint16)
        assert_same(_gather(pviews[N // 3][p], e), want, "bf16", f"all-gather param {p}")


def _bf16_nearest(x):
    """float64 -> bf16 bits with one rounding to nearest even: float64 -> fp32 rounded to
    odd (truncate, then set the last bit if inexact), then fp32 -> bf16; fp32 keeps more
    than two bits beyond bf16, so the two steps round like one (Boldo and Melquiond)."""
    from oracle.numerics import f32_to_bf16
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    over = np.abs(f.astype(np.float64)) > np.abs(x)
    f = np.where(over, np.nextafter(f, np.float32(0)), f).astype(np.float32)
    bits = f.view(np.uint32).copy()
    bits[f.astype(np.float64) != x] |= np.uint32(1)
    return f32_to_bf16(bits.view(np.float32))


def _scaled_error(got, vals_f64, N):
    """|got - exact mean| / (sum|x| / N): the error relative to the size of the
    terms, meaningful also where the mean itself cancels to near zero."""
    exact = vals_f64.sum(axis=0) / N
    scale = np.maximum(np.abs(vals_f64).sum(axis=0) / N, 1e-300)
    return np.abs(np.asarray(got, dtype=np.float64) - exact) / scale, exact


def test_wire_bf16_ring_error_study():
    """The ring that forwards bf16 partials against the one that keeps fp32
    partials, at the full sizes: the 8 x 64 MiB bf16 all-reduce (avg) and the
    64-rank FSDP layer reduce-scatter (avg, bf16 -> fp32).  Both orders are
    bit-exact against the oracle on sampled outputs; their errors against the
    exact mean (float64 sums of the bf16 inputs, exact at these magnitudes) are
    printed, and the wire ring's must be the larger."""
    from oracle.numerics import bf16_to_f32
    cfg = WORKLOADS["ar_bf16_n8"]
    N, S = cfg["nranks"], cfg["count"]
    keys = [G.stream_key(SEED, r, 0) for r in range(N)]
    arena = gc.RankArena(N)
    send = arena.alloc(S, "bf16")
    for r in range(N):
        GD.fill_normal_bf16(send[r], keys[r], cfg["sigma"])
    pos = _positions(S, N, np.random.default_rng(21), m=1 << 17)
    vals = np.stack([G.normal_bf16(keys[i], pos, cfg["sigma"]) for i in range(N)])
    wide = bf16_to_f32(vals).astype(np.float64)
    stats = {}
    for order in ("ring", "ring_wire"):
        recv = arena.alloc(S, "bf16")
        gc.gc_all_reduce(send, recv, op="avg", order=order)
        torch.cuda.synchronize()
        got = _gather(recv[N // 2], pos)
        assert_same(got, SM.all_reduce_at(vals, pos, S, "bf16", "avg", order), "bf16", f"all-reduce {order}")
        err, exact = _scaled_error(bf16_to_f32(got), wide, N)
        off = float(np.mean(_bf16_nearest(exact) != got))         # vs the exact mean rounded once
        stats[order] = (off, float(np.median(err)), float(np.quantile(err, 0.99)), float(err.max()))
        print(f"ar_bf16_n8 {order}: differs from the correctly rounded mean {off:.4%}; error / mean|x|: "
              f"median {stats[order][1]:.3e}, p99 {stats[order][2]:.3e}, max {stats[order][3]:.3e} "
              f"({len(pos)} samples)", flush=True)
    assert stats["ring_wire"][1] > stats["ring"][1] and stats["ring_wire"][0] > stats["ring"][0]
    del send, recv, arena                                     # release the 8-rank arena before the 64-rank one
    torch.cuda.empty_cache()

    N = WORKLOADS["fsdp_layer_n64"]["nranks"]
    numels = [n for _, n in fsdp_layer_tensors()]
    _, _, S, _ = OB.flat_param_shards(numels, N)
    rc = S // N
    gkeys = [G.stream_key(SEED, r, 0) for r in range(N)]
    arena = gc.RankArena(N)
    grads = arena.alloc(S, "bf16")
    for r in range(N):
        GD.fill_normal_bf16(grads[r], gkeys[r], 1e-3)
    rng = np.random.default_rng(22)
    owners = list(range(0, N, 9))
    ks = {j: np.unique(rng.integers(0, rc, size=4096)) for j in owners}
    vals = {j: np.stack([G.normal_bf16(gkeys[i], j * rc + ks[j], 1e-3) for i in range(N)]) for j in owners}
    for order in ("ring", "ring_wire"):
        shards = arena.alloc(rc, "fp32")
        gc.gc_reduce_scatter(grads, shards, op="avg", order=order)
        torch.cuda.synchronize()
        rel = []
        for j in owners:
            want = SM.reduce_scatter_at(vals[j], np.full(len(ks[j]), j), ks[j], rc, "bf16", "fp32", "avg", order)
            got = _gather(shards[j], ks[j])
            assert_same(got, want, "fp32", f"reduce-scatter {order} owner {j}")
            rel.append(_scaled_error(got, bf16_to_f32(vals[j]).astype(np.float64), N)[0])
        rel = np.concatenate(rel)
        stats[order + "64"] = (float(np.median(rel)), float(np.quantile(rel, 0.99)), float(rel.max()))
        print(f"fsdp_layer_n64 {order}: error / mean|x|: median {stats[order + '64'][0]:.3e}, "
              f"p99 {stats[order + '64'][1]:.3e}, max {stats[order + '64'][2]:.3e} ({len(rel)} samples)", flush=True)
    assert stats["ring_wire64"][0] > 10 * stats["ring64"][0] and stats["ring_wire64"][2] > stats["ring64"][2]


def _cells(count, S, R, chunk=None):
    """(i, h, lo, hi) of every cell of the two-level schedule: chunk i of S, cross-group piece h of R."""
    c1 = chunk if chunk is not None else -(-count // S)
    out = []
    for i in range(S):
        lo, hi = min(count, i * c1), min(count, (i + 1) * c1)
        c2 = max(1, -(-(hi - lo) // R))
        for h in range(R):
            a, b = lo + min(hi - lo, h * c2), lo + min(hi - lo, (h + 1) * c2)
            if a < b:
                out.append((i, h, a, b))
    return out


def test_hier_ar_n16_and_hsdp_layer_full():
    """Two nodes of eight (AIG6 §6.3.6's HSDP example) at full size: the
    two-level all-reduce of 16 x 64 MiB bf16 (avg) and the HSDP reduce-scatter
    of one transformer layer (bf16 -> fp32 avg), every output compared with the
    oracle's two-level fold cell by cell (plus a sample against host-regenerated
    inputs); every rank's all-reduce result is identical and the shard each
    group holds is the same."""
    cfg = WORKLOADS["hier_ar_n16"]
    N, S, count = cfg["nranks"], cfg["group"], cfg["count"]
    R = N // S
    keys = [G.stream_key(SEED, r, 0) for r in range(N)]
    arena = gc.RankArena(N, stagger_bytes=cfg["stagger"])          # the layout bench.py times
    send = arena.alloc(count, "bf16")
    for r in range(N):
        GD.fill_normal_bf16(send[r], keys[r], cfg["sigma"])
    recv = arena.alloc(count, "bf16")
    gc.gc_hier_all_reduce(send, recv, S, op="avg", order="ring")
    torch.cuda.synchronize()
    for r in range(1, N):
        assert torch.equal(recv[r].view(torch.int16), recv[0].view(torch.int16)), f"rank {r} differs"
    c1 = -(-count // S)
    edges = []
    for i in range(S):
        lo = i * c1
        L = min(count, lo + c1) - lo
        c2 = -(-L // R)
        for h in range(R):
            a, b = lo + min(L, h * c2), lo + min(L, (h + 1) * c2)
            edges += [a, a + 1, b - 2, b - 1]
    pos = np.unique(np.concatenate([np.random.default_rng(31).integers(0, count, size=1 << 14), edges]))
    pos = pos[(pos >= 0) & (pos < count)]
    vals = np.stack([G.normal_bf16(keys[r], pos, cfg["sigma"]) for r in range(N)])
    g0, m0 = SM.hier_fold_starts(pos, count, S, R, "ring")
    want = SM.hier_reduce_positions(vals, S, g0, m0, "bf16", "avg", "bf16")
    assert_same(_gather(recv[5], pos), want, "bf16", "two-level all-reduce")
    for i, h, a, b in _cells(count, S, R):                     # every output, cell by cell
        want = SM.hier_reduce_block(_slices(send, a, b), S, (h + 1) % R, (i + 1) % S, "bf16", "avg", "bf16")
        assert_same(from_dev(recv[5][a:b]), want, "bf16", f"two-level cell ({i}, {h})")
    del send, recv, arena                                     # release the first arena before the second
    torch.cuda.empty_cache()

    numels = [n for _, n in fsdp_layer_tensors()]
    _, _, Sflat, _ = OB.flat_param_shards(numels, S)
    rc = Sflat // S
    arena = gc.RankArena(N, stagger_bytes=WORKLOADS["hsdp_layer_n16"]["stagger"])
    grads = arena.alloc(Sflat, "bf16")
    for r in range(N):
        GD.fill_normal_bf16(grads[r], keys[r], 1e-3)
    shards = arena.alloc(rc, "fp32")
    gc.gc_hsdp_reduce_scatter(grads, shards, S, op="avg", order="ring")
    torch.cuda.synchronize()
    for i in range(S):
        for g in range(1, R):
            assert torch.equal(shards[g * S + i], shards[i]), f"member {i} group {g}"
    rng = np.random.default_rng(32)
    for i in (0, 3, S - 1):
        k = np.unique(np.concatenate([rng.integers(0, rc, size=4096), [0, rc - 1]]))
        p = i * rc + k
        vals = np.stack([G.normal_bf16(keys[r], p, 1e-3) for r in range(N)])
        g0, m0 = SM.hier_fold_starts(p, Sflat, S, R, "ring", chunk=rc)
        want = SM.hier_reduce_positions(vals, S, g0, m0, "bf16", "avg", "fp32")
        assert_same(_gather(shards[S + i], k), want, "fp32", f"hsdp member {i}")
    for i, h, a, b in _cells(Sflat, S, R, chunk=rc):           # every output, cell by cell
        want = SM.hier_reduce_block(_slices(grads, a, b), S, (h + 1) % R, (i + 1) % S, "bf16", "avg", "fp32")
        assert_same(from_dev(shards[S + i][a - i * rc:b - i * rc]), want, "fp32", f"hsdp cell ({i}, {h})")


def test_wire_bf16_error_study_ddp_and_hsdp():
    """The bf16-wire ring against the fp32-partial ring on two more paths at
    full size: the DDP step's 226 zero-copy bucket all-reduces of the Llama-7B
    gradient set (8 ranks, avg) and the HSDP reduce-scatter of one layer on 2 x 8
    ranks (avg, bf16 -> fp32).  Sampled outputs of both orders are bit-exact
    against the oracle's folds in that order; the errors against the exact mean
    are printed, and the wire's must be the larger (DTLM §11)."""
    from oracle.numerics import bf16_to_f32
    cfg = WORKLOADS["ddp_llama7b"]
    N, sigma, cap = cfg["nranks"], cfg["sigma"], cfg["cap_bytes"]
    numels, offs = _llama_layout()
    total = int(offs[-1])
    keys = [G.stream_key(SEED, r, 0) for r in range(N)]
    arena = gc.RankArena(N, min_bytes=total * 2 + (1 << 30))
    flat = arena.alloc(total, "bf16")
    tensors = [flat[r][int(offs[t]):int(offs[t]) + numels[t]] for r in range(N) for t in range(len(numels))]
    ptrs = gc.gc_pointers(tensors)
    plan = gc.BucketPlan(numels, "bf16", cap, reverse=True)
    oracle_buckets = OB.assign_buckets(numels, 2, cap, reverse=True)
    rng = np.random.default_rng(23)
    samples = []                                    # (bucket positions, model-order flat indices, used)
    for ts in oracle_buckets:
        boffs, used, _ = OB.bucket_layout(ts, numels)
        e = np.unique(np.concatenate([rng.integers(0, used, size=256), [0, used - 1]]))
        which = np.searchsorted(np.asarray(boffs), e, side="right") - 1
        samples.append((e, np.array([offs[ts[w]] + (ee - boffs[w]) for w, ee in zip(which, e)], np.int64), used))
    vals = [np.stack([G.normal_bf16(keys[r], f, sigma) for r in range(N)]) for _, f, _ in samples]
    stats = {}
    for order in ("ring", "ring_wire"):
        for r in range(N):                          # fresh gradients: the all-reduce runs in place
            GD.fill_normal_bf16(flat[r], keys[r], sigma)
        for b in range(plan.nbuckets):
            plan.all_reduce(b, ptrs, N, op="avg", order=order)
        torch.cuda.synchronize()
        got = _gather(flat[6], np.concatenate([f for _, f, _ in samples]))
        want = np.concatenate([SM.all_reduce_at(v, e, used, "bf16", "avg", order)
                               for v, (e, _, used) in zip(vals, samples)])
        assert_same(got, want, "bf16", f"ddp bucket all-reduce {order}")
        wide = np.concatenate([bf16_to_f32(v).astype(np.float64) for v in vals], axis=1)
        err, exact = _scaled_error(bf16_to_f32(got), wide, N)
        off = float(np.mean(_bf16_nearest(exact) != got))
        stats[order] = (off, float(np.median(err)), float(np.quantile(err, 0.99)), float(err.max()))
        print(f"ddp_llama7b zero-copy {order}: differs from the correctly rounded mean {off:.4%}; error / mean|x|: "
              f"median {stats[order][1]:.3e}, p99 {stats[order][2]:.3e}, max {stats[order][3]:.3e} "
              f"({len(got)} samples over {plan.nbuckets} buckets)", flush=True)
    assert stats["ring_wire"][1] > stats["ring"][1] and stats["ring_wire"][0] > stats["ring"][0]
    plan.close()
    del flat, tensors, ptrs, arena
    torch.cuda.empty_cache()

    hc = WORKLOADS["hsdp_layer_n16"]
    N, S = hc["nranks"], hc["group"]
    R = N // S
    _, _, Sflat, _ = OB.flat_param_shards([n for _, n in fsdp_layer_tensors()], S)
    rc = Sflat // S
    keys = [G.stream_key(SEED, r, 0) for r in range(N)]
    arena = gc.RankArena(N, stagger_bytes=hc["stagger"])
    grads = arena.alloc(Sflat, "bf16")
    for r in range(N):
        GD.fill_normal_bf16(grads[r], keys[r], hc["grad_sigma"])
    cells = [(i, h, a, b) for i, h, a, b in _cells(Sflat, S, R, chunk=rc)]
    pos = [np.unique(np.concatenate([rng.integers(a, b, size=1024), [a, b - 1]])) for _, _, a, b in cells]
    cvals = [np.stack([G.normal_bf16(keys[r], p, hc["grad_sigma"]) for r in range(N)]) for p in pos]
    for order in ("ring", "ring_wire"):
        shards = arena.alloc(rc, "fp32")
        gc.gc_hsdp_reduce_scatter(grads, shards, S, op="avg", order=order)
        torch.cuda.synchronize()
        rel = []
        for (i, h, a, b), p, v in zip(cells, pos, cvals):
            want = SM.hier_reduce_block(list(v), S, (h + 1) % R, (i + 1) % S, "bf16", "avg", "fp32",
                                        "bf16" if order == "ring_wire" else None)
            got = _gather(shards[S + i], p - i * rc)
            assert_same(got, want, "fp32", f"hsdp {order} cell ({i}, {h})")
            rel.append(_scaled_error(got, bf16_to_f32(v).astype(np.float64), N)[0])
        rel = np.concatenate(rel)
        stats["hsdp_" + order] = (float(np.median(rel)), float(np.quantile(rel, 0.99)), float(rel.max()))
        print(f"hsdp_layer_n16 {order}: error / mean|x|: median {stats['hsdp_' + order][0]:.3e}, "
              f"p99 {stats['hsdp_' + order][1]:.3e}, max {stats['hsdp_' + order][2]:.3e} ({len(rel)} samples)",
              flush=True)
    assert stats["hsdp_ring_wire"][0] > 10 * stats["hsdp_ring"][0]
