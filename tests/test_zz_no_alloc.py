"""gc_moe_route_noalloc, the routing plan for callers that cannot allocate
device memory, against gc_moe_route (the same plan with caller scratch) through
the C ABI: bit-identical splits and (rank, row) tables on two calls in a row,
the second with a smaller input (the library's static scratch keeps the first
call's contents), both also equal to the oracle's plan; a plan larger than the
static scratch is refused before anything is launched."""

import numpy as np
import pytest
import torch

import collective_communication_reduction_amd as gc
from gen.workloads import route_tokens
from oracle import moe as M
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32).reshape(-1))).to(DEV)


def _plan(route_fn, experts, N, E, K, **kw):
    ntok = [len(e) for e in experts]
    splits = torch.full((N * N * E,), -7, dtype=torch.int64, device=DEV)
    dest = [torch.full((max(1, n * K * 2),), -7, dtype=torch.int32, device=DEV) for n in ntok]
    route_fn([_i32(e) for e in experts], ntok, K, E, splits, dest, **kw)
    torch.cuda.synchronize()
    return splits.cpu().numpy(), [d.cpu().numpy() for d in dest]


def _with_scratch(experts, ntok, K, E, splits, dest):
    scratch = torch.empty(max(1, gc.gc_moe_route_scratch_bytes(ntok, K, E)), dtype=torch.uint8, device=DEV)
    gc.gc_moe_route(experts, ntok, K, E, splits, dest, scratch)


@pytest.mark.parametrize("N,E,T,K,seed", [(8, 8, 3000, 2, 3), (4, 3, 700, 2, 4)])
def test_noalloc_route_equals_route_twice(N, E, T, K, seed):
    # first call at T tokens per source, then a smaller one (ragged, one empty source)
    sizes = [[T] * N, [max(0, T // 5 - 37 * s) for s in range(N - 1)] + [0]]
    for call, ts in enumerate(sizes):
        experts = [route_tokens(seed + call, s, t, N * E, K, 1.1) if t else np.zeros((0, K), np.int64)
                   for s, t in enumerate(ts)]
        got_s, got_d = _plan(gc.gc_moe_route_noalloc, experts, N, E, K)
        ref_s, ref_d = _plan(_with_scratch, experts, N, E, K)
        assert np.array_equal(got_s, ref_s), f"call {call}: splits"
        for s in range(N):
            assert np.array_equal(got_d[s], ref_d[s]), f"call {call}: source {s}"
        want_splits, dr, dw = M.route_plan(experts, N, E)
        assert np.array_equal(got_s.reshape(N, N, E), want_splits)
        for s in range(N):
            d = got_d[s][:2 * ts[s] * K].reshape(-1, 2)
            assert np.array_equal(d[:, 0], dr[s]) and np.array_equal(d[:, 1], dw[s]), f"call {call}: source {s}"


def test_noalloc_route_refuses_plans_beyond_its_scratch():
    N, E, K = 8, 64, 8                                   # 512 bins: 2 KiB of counts per tile of 1024 routes
    ntok = [300_000] * N
    assert gc.gc_moe_route_scratch_bytes(ntok, K, E) > gc.GC_MOE_ROUTE_NOALLOC_SCRATCH_BYTES
    splits = torch.empty(N * N * E, dtype=torch.int64, device=DEV)
    experts = [torch.empty(1, dtype=torch.int32, device=DEV)] * N   # never read: refused on the host
    dest = [torch.empty(1, dtype=torch.int32, device=DEV)] * N
    ptr = gc.gc_pointers
    with pytest.raises(gc.GcError) as e:
        gc.gc_moe_route_noalloc(ptr(experts), ntok, K, E, splits, ptr(dest))
    assert e.value.status == gc.GC_ERR_UNSUPPORTED
