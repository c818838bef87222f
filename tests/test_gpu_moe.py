"""GPU parity of the MoE routing plan, dispatch and combine against the oracle
(DTLM §8), element by element on seeded inputs: ragged and empty sources,
several tiles of routes, one to eight experts per token, dropped routes, row
sizes that take the 16-byte, 4-, 2- and 1-byte paths, and special values."""

import numpy as np
import pytest
import torch

import collective_communication_reduction_amd as gc
from gen.workloads import route_tokens
from oracle import moe as M
from oracle.numerics import f32_to_bf16
from tests.gpu_util import DEV, assert_same, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32).reshape(-1))).to(DEV)


def _routing(rng, N, E, T, K, drop=0.0):
    """Top-K distinct experts per token; a fraction `drop` of routes get ids outside the range."""
    out = []
    for Ts in T:
        ex = np.argsort(rng.random((Ts, N * E)), axis=1)[:, :K].astype(np.int64)
        if drop:
            m = rng.random(ex.shape) < drop
            ex[m] = rng.choice([-1, N * E, 1 << 20], size=int(m.sum()))
        out.append(ex)
    return out


def route_on_device(experts, N, E, K):
    ntok = [len(e) for e in experts]
    splits = torch.full((N * N * E,), -7, dtype=torch.int64, device=DEV)
    dest = [torch.full((max(1, n * K * 2),), -7, dtype=torch.int32, device=DEV) for n in ntok]
    scratch = torch.empty(max(1, gc.gc_moe_route_scratch_bytes(ntok, K, E)), dtype=torch.uint8, device=DEV)
    gc.gc_moe_route([_i32(e) for e in experts], ntok, K, E, splits, dest, scratch)
    return ntok, splits, dest


def check_plan(experts, N, E, K, splits, dest):
    want_splits, dr, dw = M.route_plan(experts, N, E)
    torch.cuda.synchronize()
    assert np.array_equal(splits.cpu().numpy().reshape(N, N, E), want_splits)
    for s in range(N):
        n = len(experts[s]) * K
        got = dest[s].cpu().numpy()[:2 * n].reshape(-1, 2)
        assert np.array_equal(got[:, 0], dr[s]), f"source {s} ranks"
        assert np.array_equal(got[:, 1], dw[s]), f"source {s} rows"
    return want_splits


ROUTE_CASES = [
    # N, E, tokens per source, K, drop fraction
    (1, 1, [5], 1, 0.0),
    (2, 2, [3, 3], 2, 0.0),
    (4, 3, [7, 0, 1100, 1], 2, 0.0),          # ragged, one empty source, 5 tiles of 512 routes
    (3, 5, [300, 301, 299], 3, 0.0),
    (8, 8, [2000] * 8, 2, 0.0),
    (8, 8, [600] * 8, 8, 0.1),                # eight routes per token, dropped routes
    (64, 2, [50 if s % 5 else 0 for s in range(64)], 1, 0.0),
    (2, 4096, [700, 5], 8, 0.0),              # 8192 experts: tiles of 8192 routes
]


@pytest.mark.parametrize("N,E,T,K,drop", ROUTE_CASES)
def test_route_plan(N, E, T, K, drop):
    rng = np.random.default_rng(N * 100 + K)
    experts = _routing(rng, N, E, T, K, drop)
    _, splits, dest = route_on_device(experts, N, E, K)
    check_plan(experts, N, E, K, splits, dest)


def test_route_plan_worked_example(golden):
    lines = golden("moe_route_n2.txt")
    experts = [np.zeros((3, 2), dtype=np.int64) for _ in range(2)]
    for l in lines:
        if l[0] == "route":
            experts[int(l[1])][int(l[2]), int(l[3])] = int(l[4])
    _, splits, dest = route_on_device(experts, 2, 2, 2)
    torch.cuda.synchronize()
    for l in lines:
        if l[0] == "route":
            s, t, k, _, d, r = map(int, l[1:])
            assert dest[s].cpu().numpy().reshape(-1, 2)[t * 2 + k].tolist() == [d, r]
        if l[0] == "split":
            s, d, e, n = map(int, l[1:])
            assert int(splits[(s * 2 + d) * 2 + e]) == n


def test_route_plan_zipf_routing():
    N, E, T, K = 8, 8, 3000, 2
    experts = [route_tokens(3, s, T, N * E, K, 1.1) for s in range(N)]
    _, splits, dest = route_on_device(experts, N, E, K)
    check_plan(experts, N, E, K, splits, dest)


def _byte_rows(rng, n, row_bytes):
    return rng.integers(0, 256, size=n * row_bytes).astype(np.uint8)


@pytest.mark.parametrize("row_bytes,offset", [(8192, 0), (2048, 0), (48, 0), (16, 0), (64, 4), (12, 0),
                                              (6, 0), (5, 0), (8192, 2), (4112, 0)])
def test_dispatch(row_bytes, offset):
    rng = np.random.default_rng(row_bytes + offset)
    N, E, K = 4, 2, 2
    T = [37, 0, 64, 5]
    experts = _routing(rng, N, E, T, K, drop=0.05)
    ntok, splits, dest = route_on_device(experts, N, E, K)
    want_splits = check_plan(experts, N, E, K, splits, dest)
    tokens = [_byte_rows(rng, t, row_bytes) for t in T]
    want = M.dispatch(tokens, experts, N, E, row_bytes)
    rows = want_splits.sum(axis=(0, 2))
    spare = 3                                  # rows past the plan stay untouched
    tok_dev = [torch.from_numpy(np.concatenate([np.zeros(offset, np.uint8), t])).to(DEV)[offset:] for t in tokens]
    recv_full = [torch.full((offset + (int(r) + spare) * row_bytes,), 0xA5, dtype=torch.uint8, device=DEV)
                 for r in rows]
    recv = [b[offset:] for b in recv_full]
    gc.gc_moe_dispatch(tok_dev, ntok, dest, K, row_bytes, recv, [int(r) + spare for r in rows])
    torch.cuda.synchronize()
    for d in range(N):
        got = from_dev(recv[d])
        n = int(rows[d]) * row_bytes
        assert np.array_equal(got[:n], want[d]), f"rank {d}"
        assert np.all(got[n:] == 0xA5), f"rank {d} wrote past its rows"


@pytest.mark.parametrize("K", [1, 3, 5])
@pytest.mark.parametrize("row_bytes", [8192, 4100, 1001, 48])
def test_dispatch_topk(K, row_bytes):
    """Routes per token with and without a compiled-in count (1 and 2 are; 3 and 5
    go through batches of four), on rows a wavefront shares (8192: 16-byte
    units; 4100: 4-byte units; 1001: 1-byte units) and on rows several share a
    wavefront (48)."""
    rng = np.random.default_rng(1000 * K + row_bytes)
    N, E = 3, 4
    T = [41, 7, 0]
    experts = _routing(rng, N, E, T, K, drop=0.1)
    ntok, splits, dest = route_on_device(experts, N, E, K)
    want_splits = check_plan(experts, N, E, K, splits, dest)
    tokens = [_byte_rows(rng, t, row_bytes) for t in T]
    want = M.dispatch(tokens, experts, N, E, row_bytes)
    rows = want_splits.sum(axis=(0, 2))
    tok_dev = [torch.from_numpy(t).to(DEV) if t.size else torch.zeros(16, dtype=torch.uint8, device=DEV)
               for t in tokens]
    recv = [torch.full((max(16, (int(r) + 2) * row_bytes),), 0x5A, dtype=torch.uint8, device=DEV) for r in rows]
    gc.gc_moe_dispatch(tok_dev, ntok, dest, K, row_bytes, recv, [int(r) + 2 for r in rows])
    torch.cuda.synchronize()
    for d in range(N):
        got = from_dev(recv[d])
        n = int(rows[d]) * row_bytes
        assert np.array_equal(got[:n], want[d]), f"rank {d}"
        assert np.all(got[n:] == 0x5A), f"rank {d} wrote past its rows"


def _expert_rows(rng, n, hidden, dtype, special):
    x = rng.normal(size=n * hidden).astype(np.float32)
    if special and x.size >= 8:
        x[:6] = [np.inf, -np.inf, np.nan, 1e-40, -0.0, 3e38]
    return f32_to_bf16(x) if dtype == "bf16" else x


COMBINE_CASES = [
    # dtype, hidden, K, drop
    ("bf16", 4096, 2, 0.0),
    ("bf16", 1000, 2, 0.05),        # 2000-byte rows: 16-byte units, odd unit count
    ("bf16", 7, 1, 0.0),            # 14-byte rows: element path
    ("bf16", 64, 3, 0.1),           # K with no compiled-in specialisation
    ("fp32", 999, 2, 0.0),          # element path
    ("fp32", 1024, 8, 0.2),
    ("fp32", 4, 1, 0.0),            # one 16-byte unit per row
    ("bf16", 4099, 2, 0.05),        # element path, rows shared by five workgroups (column blocks)
]


@pytest.mark.parametrize("dtype,hidden,K,drop", COMBINE_CASES)
def test_combine(dtype, hidden, K, drop):
    rng = np.random.default_rng(hidden * 10 + K)
    N, E = 4, 3
    T = [29, 3, 0, 70]
    experts = _routing(rng, N, E, T, K, drop)
    ntok, splits, dest = route_on_device(experts, N, E, K)
    want_splits = check_plan(experts, N, E, K, splits, dest)
    rows = want_splits.sum(axis=(0, 2))
    y = [_expert_rows(rng, int(r), hidden, dtype, special=True) for r in rows]
    w = [rng.normal(size=(t, K)).astype(np.float32) for t in T]
    for ws in w:
        if ws.size > 4:
            ws.reshape(-1)[:3] = [0.0, -1.0, np.float32(2.0 ** -130)]
    want = M.combine(y, experts, w, N, E, hidden, dtype)
    y_dev = [to_dev(a, dtype) for a in y]
    w_dev = [torch.from_numpy(ws.reshape(-1)).to(DEV) for ws in w]
    # each output is a view with 64 sentinel elements after it: nothing past a source's rows may be written
    out_full = [torch.full((t * hidden + 64,), 7.0, dtype=y_dev[0].dtype, device=DEV) for t in T]
    out = [o[:t * hidden] for o, t in zip(out_full, T)]
    gc.gc_moe_combine(y_dev, [int(r) for r in rows], dest, w_dev, ntok, K, hidden, dtype, out)
    torch.cuda.synchronize()
    for s in range(N):
        assert_same(from_dev(out[s]), want[s], dtype, f"source {s}")
        tail = out_full[s][T[s] * hidden:]
        assert torch.equal(tail, torch.full_like(tail, 7.0)), f"source {s}: written past its rows"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_dispatch_then_combine_round_trip(dtype):
    """Route, dispatch from token order, identity experts, combine: against the
    oracle's own dispatch feeding its combine."""
    rng = np.random.default_rng(17)
    N, E, K, H = 8, 8, 2, 256
    T = [100 + 13 * s for s in range(N)]
    experts = [route_tokens(5, s, T[s], N * E, K, 1.1) for s in range(N)]
    ntok, splits, dest = route_on_device(experts, N, E, K)
    want_splits = check_plan(experts, N, E, K, splits, dest)
    rows = [int(r) for r in want_splits.sum(axis=(0, 2))]
    tokens = [_expert_rows(rng, t, H, dtype, special=False) for t in T]
    w = [rng.random((t, K)).astype(np.float32) for t in T]
    want = M.combine(M.dispatch(tokens, experts, N, E, H), experts, w, N, E, H, dtype)
    tok_dev = [to_dev(t, dtype) for t in tokens]
    es = 2 if dtype == "bf16" else 4
    recv = [torch.empty(max(1, r * H), dtype=tok_dev[0].dtype, device=DEV) for r in rows]
    gc.gc_moe_dispatch(tok_dev, ntok, dest, K, H * es, recv, rows)
    out = [torch.empty(t * H, dtype=tok_dev[0].dtype, device=DEV) for t in T]
    gc.gc_moe_combine(recv, rows, dest, [torch.from_numpy(x.reshape(-1)).to(DEV) for x in w], ntok, K, H, dtype, out)
    torch.cuda.synchronize()
    for s in range(N):
        assert_same(from_dev(out[s]), want[s], dtype, f"source {s}")


@pytest.mark.parametrize("H", [8, 1024])
def test_malformed_plan_entries_are_skipped(H):
    """Entries naming a rank or row outside the buffers are skipped, not followed.
    H = 1024 fp32 (4 KiB rows) puts whole wavefronts on one row, where the
    dispatch reads each entry once per wavefront."""
    N, K = 2, 2
    dest = [_i32([[0, 0], [5, 0], [1, 1], [1, 99], [-1, 0], [0, -3]]), _i32([[1, 0], [0, 1]])]
    ntok = [3, 1]
    tokens = [torch.arange(3 * H, dtype=torch.float32, device=DEV) + 1, torch.full((H,), -1.0, device=DEV)]
    recv = [torch.zeros(2 * H, device=DEV), torch.zeros(2 * H, device=DEV)]
    gc.gc_moe_dispatch(tokens, ntok, dest, K, H * 4, recv, [2, 2])
    torch.cuda.synchronize()
    r0, r1 = recv[0].cpu().numpy().reshape(2, H), recv[1].cpu().numpy().reshape(2, H)
    assert np.array_equal(r0[0], np.arange(1, H + 1)) and np.all(r0[1] == -1.0)
    assert np.all(r1[0] == -1.0) and np.array_equal(r1[1], np.arange(H + 1, 2 * H + 1))
    w = [torch.full((6,), 0.5, device=DEV), torch.ones(2, device=DEV)]
    out = [torch.full((3 * H,), 9.0, device=DEV), torch.full((H,), 9.0, device=DEV)]
    gc.gc_moe_combine(recv, [2, 2], dest, w, ntok, K, H, "fp32", out)
    torch.cuda.synchronize()
    o0 = out[0].cpu().numpy().reshape(3, H)
    assert np.array_equal(o0[0], 0.5 * np.arange(1, H + 1))          # only the first route is kept
    assert np.array_equal(o0[1], 0.5 * np.arange(H + 1, 2 * H + 1))
    assert np.all(o0[2] == 0.0) and not np.signbit(o0[2]).any()       # no route kept: zeros
    assert np.array_equal(out[1].cpu().numpy(), r1[0] + r0[1])


@pytest.mark.parametrize("N,E,K,H,dtype", [(64, 2, 2, 96, "bf16"), (64, 1, 3, 5, "fp32"), (16, 4, 8, 1, "bf16")])
def test_many_ranks_round_trip(N, E, K, H, dtype):
    """The 64-rank argument layout, three and eight routes per token, and rows
    of one element."""
    rng = np.random.default_rng(N * K + H)
    T = [int(x) for x in rng.integers(0, 40, size=N)]
    experts = _routing(rng, N, E, T, K, drop=0.05)
    ntok, splits, dest = route_on_device(experts, N, E, K)
    want_splits = check_plan(experts, N, E, K, splits, dest)
    rows = [int(r) for r in want_splits.sum(axis=(0, 2))]
    tokens = [_expert_rows(rng, t, H, dtype, special=False) for t in T]
    w = [rng.normal(size=(t, K)).astype(np.float32) for t in T]
    want = M.combine(M.dispatch(tokens, experts, N, E, H), experts, w, N, E, H, dtype)
    tok_dev = [to_dev(t, dtype) if t.size else 0 for t in tokens]
    es = 2 if dtype == "bf16" else 4
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    recv = [torch.empty(max(1, r * H), dtype=tdt, device=DEV) for r in rows]
    gc.gc_moe_dispatch(tok_dev, ntok, dest, K, H * es, recv, rows)
    out = [torch.empty(max(1, t * H), dtype=tdt, device=DEV) for t in T]
    w_dev = [torch.from_numpy(x.reshape(-1)).to(DEV) if x.size else 0 for x in w]
    gc.gc_moe_combine(recv, rows, dest, w_dev, ntok, K, H, dtype, out)
    torch.cuda.synchronize()
    for s in range(N):
        if T[s]:
            assert_same(from_dev(out[s])[:T[s] * H], want[s], dtype, f"source {s}")
