"""CPU tests of the C ABI: the library loads, exports every declared call, and
rejects bad arguments on the host before anything is launched (no GPU needed:
every call here returns before the first HIP call).  The host-side bucket
planner is compared with the oracle's independent planner."""

import ctypes
import os
import re

import pytest

import collective_communication_reduction_amd as gc
from gen.workloads import fsdp_layer_tensors, llama7b_tensors
from oracle import buckets as OB

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # a host-side stand-in address; never dereferenced by these calls


def _declared():
    text = open(os.path.join(ROOT, "include", "gc.h"), encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gc_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 12
    lib = ctypes.CDLL(gc.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    assert gc.gc_status_string(gc.GC_OK) == "GC_OK"
    assert gc.gc_status_string(gc.GC_ERR_UNSUPPORTED) == "GC_ERR_UNSUPPORTED"
    assert gc.gc_version() >= 100


def _ptrs(n, step=1 << 30, base=FAKE):
    return [base + i * step for i in range(n)]


def _status(fn, *a, **k):
    try:
        fn(*a, **k)
    except gc.GcError as e:
        return e.status
    return gc.GC_OK


def test_all_reduce_validation():
    ar = gc.gc_all_reduce
    s, r = _ptrs(4), _ptrs(4, base=FAKE + (1 << 40))
    assert _status(ar, s, r, count=0, dtype="bf16", stream=0) == gc.GC_OK          # nothing to do
    assert _status(ar, [], [], count=8, dtype="bf16", stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(ar, _ptrs(65), _ptrs(65, base=FAKE + (1 << 41)), count=8, dtype="bf16",
                   stream=0) == gc.GC_ERR_UNSUPPORTED
    assert _status(ar, s, r, count=8, dtype="int32", op="avg", stream=0) == gc.GC_ERR_UNSUPPORTED
    assert _status(ar, s, r, count=8, dtype=7, stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(ar, s, r, count=8, dtype="fp32", op=9, stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(ar, s[:3] + [0], r, count=8, dtype="fp32", stream=0) == gc.GC_ERR_INVALID_ARG   # null
    assert _status(ar, s[:3] + [FAKE + 2], r, count=8, dtype="fp32", stream=0) == gc.GC_ERR_INVALID_ARG  # misaligned
    # overlapping outputs, and an output partially overlapping an input
    assert _status(ar, s, r[:3] + [r[2] + 16], count=8, dtype="fp32", stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(ar, s, r[:3] + [s[0] + 4], count=8, dtype="fp32", stream=0) == gc.GC_ERR_INVALID_ARG
    # RS_AG needs enough scratch, disjoint from the buffers
    need = gc.gc_all_reduce_scratch_bytes(1000, 4, "bf16")
    assert need >= 2000 and need % 256 == 0
    assert gc.gc_all_reduce_scratch_bytes(1000, 4, "bf16", "fused") == 0
    assert _status(ar, s, r, count=1000, dtype="bf16", algo="rs_ag", scratch=FAKE + (1 << 42),
                   scratch_bytes=need - 1, stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(ar, s, r, count=1000, dtype="bf16", algo="rs_ag", scratch=s[1],
                   scratch_bytes=need, stream=0) == gc.GC_ERR_INVALID_ARG


def test_reduce_scatter_validation():
    rs = gc.gc_reduce_scatter
    s, r = _ptrs(4), _ptrs(4, base=FAKE + (1 << 40))
    kw = dict(recv_count=16, in_dtype="bf16", out_dtype="fp32", stream=0)
    assert _status(rs, s, r, recv_count=0, in_dtype="bf16", out_dtype="fp32", stream=0) == gc.GC_OK
    assert _status(rs, s, r, recv_count=16, in_dtype="int32", out_dtype="fp32", stream=0) == gc.GC_ERR_UNSUPPORTED
    assert _status(rs, s, r, op="avg", recv_count=16, in_dtype="int32", out_dtype="int32",
                   stream=0) == gc.GC_ERR_UNSUPPORTED
    # in place is only allowed with matching types: here bf16 -> fp32 sits on send
    inplace = [s[i] + i * 16 * 2 for i in range(4)]
    assert _status(rs, s, inplace, **kw) == gc.GC_ERR_INVALID_ARG
    # recv inside another rank's send buffer
    assert _status(rs, s, [s[1] + 64] + r[1:], recv_count=16, in_dtype="bf16", out_dtype="bf16",
                   stream=0) == gc.GC_ERR_INVALID_ARG


def test_all_gather_validation():
    ag = gc.gc_all_gather
    s, r = _ptrs(4), _ptrs(4, base=FAKE + (1 << 40))
    assert _status(ag, s, r, count=0, dtype="bf16", stream=0) == gc.GC_OK
    assert _status(ag, s, r[:3] + [r[0]], count=8, dtype="bf16", stream=0) == gc.GC_ERR_INVALID_ARG
    # send inside recv at the wrong slot
    assert _status(ag, [r[0] + 2 * 8 * 2] + s[1:], r, count=8, dtype="bf16", stream=0) == gc.GC_ERR_INVALID_ARG


def test_all_to_all_validation():
    a2a = gc.gc_all_to_all
    s, r = _ptrs(2), _ptrs(2, base=FAKE + (1 << 40))
    ok = [[[1], [2]], [[3], [4]]]
    assert _status(a2a, s, r, [[[0], [0]], [[0], [0]]], 16, stream=0) == gc.GC_OK      # no rows
    assert _status(a2a, s, r, [[[1], [-2]], [[3], [4]]], 16, stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(a2a, s, r, ok, 0, stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(a2a, s, [r[0], r[0] + 16], ok, 16, stream=0) == gc.GC_ERR_INVALID_ARG   # recv overlap
    assert _status(a2a, s, [r[0], s[0]], ok, 16, stream=0) == gc.GC_ERR_INVALID_ARG         # recv on send
    big = [[[1 << 31], [0]], [[0], [0]]]
    assert _status(a2a, s, r, big, 16, stream=0) == gc.GC_ERR_UNSUPPORTED


@pytest.mark.parametrize("reverse", [True, False])
def test_bucket_plan_matches_oracle_llama(reverse):
    numels = [n for _, n in llama7b_tensors()]
    cap = 25 * 1024 * 1024
    plan = gc.BucketPlan(numels, "bf16", cap, reverse=reverse)
    want = OB.assign_buckets(numels, 2, cap, reverse=reverse)
    assert plan.nbuckets == len(want)
    for b, ts in enumerate(want):
        assert plan.bucket_tensors(b) == ts
        offs, used, padded = OB.bucket_layout(ts, numels)
        assert [plan.tensor_offset[t] for t in ts] == offs
        assert plan.bucket_numel[b] == padded
    plan.close()


def test_flat_plan_matches_oracle():
    numels = [n for _, n in fsdp_layer_tensors()]
    plan = gc.BucketPlan(numels, "bf16", gc.SIZE_MAX, reverse=False, pad_to=64)
    intervals, used, padded, _ = OB.flat_param_shards(numels, 64)
    assert plan.nbuckets == 1 and plan.bucket_numel == [padded]
    assert [(plan.tensor_offset[t], plan.tensor_offset[t] + numels[t]) for t in range(len(numels))] == intervals
    odd = gc.BucketPlan([6, 2, 4, 2], "bf16", gc.SIZE_MAX, reverse=False, pad_to=4)
    assert odd.bucket_numel == [16]


def test_bucket_plan_small_rules():
    assert gc.BucketPlan([10, 10, 10], "bf16", 15 * 2, reverse=False).nbuckets == 2
    p = gc.BucketPlan([5, 100, 5], "bf16", 50 * 2, reverse=False)
    assert [p.bucket_tensors(b) for b in range(p.nbuckets)] == [[0, 1], [2]]
    empty = gc.BucketPlan([], "bf16", 100)
    assert empty.nbuckets == 0


def test_bucket_pack_validation():
    plan = gc.BucketPlan([8, 8], "bf16", 1 << 20)
    tensors = _ptrs(4)
    bufs = _ptrs(2, base=FAKE + (1 << 40))
    assert _status(plan.pack, 5, tensors, bufs, 2, stream=0) == gc.GC_ERR_INVALID_ARG          # bad bucket
    assert _status(plan.pack, 0, tensors[:3] + [0], bufs, 2, stream=0) == gc.GC_ERR_INVALID_ARG  # null tensor
    assert _status(plan.pack, 0, tensors, [bufs[0], bufs[0] + 8], 2, stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(plan.unpack, 0, bufs, tensors, 0, stream=0) == gc.GC_ERR_INVALID_ARG
    with pytest.raises(gc.GcError):
        gc.gc_bucket_plan_create([1, 2], "bf16", 10, pad_to=0)
    with pytest.raises(gc.GcError):
        gc.gc_bucket_plan_create([1, 2], "bf16", 10, pad_to=(1 << 20) + 1)   # above the padding limit
    # a bucket whose padded bytes do not fit in 64 bits is refused
    with pytest.raises(gc.GcError):
        gc.gc_bucket_plan_create([8, (1 << 62) - 16], "fp32", gc.SIZE_MAX, pad_to=1 << 20)
    with pytest.raises(gc.GcError):
        gc.gc_bucket_plan_create([1 << 62], "bf16", gc.SIZE_MAX)


def test_extent_and_copy_volume_limits():
    """No buffer extent beyond 2^40 bytes (more than any one GPU holds) and no all-to-all moving more than
    2^42 bytes in one call: both are refused on the host, which keeps every planned tile count in 32 bits."""
    big = (1 << 39) + 8                                   # bf16 elements: 2^40 + 16 bytes
    s, r = _ptrs(2, step=1 << 41), _ptrs(2, step=1 << 41, base=FAKE + (1 << 44))
    assert _status(gc.gc_all_reduce, s, r, count=big, dtype="bf16", stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(gc.gc_reduce_scatter, s, r, recv_count=big // 2, in_dtype="bf16", out_dtype="bf16",
                   stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(gc.gc_all_gather, s, r, count=big // 2, dtype="bf16", stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(gc.gc_hier_all_reduce, _ptrs(4, step=1 << 41), _ptrs(4, step=1 << 41, base=FAKE + (1 << 44)),
                   2, count=big, dtype="bf16", stream=0) == gc.GC_ERR_INVALID_ARG
    # 8 ranks each sending 2^40 bytes (2^25 rows of 4 KiB to every rank): every buffer is possible, the
    # call's 2^43 bytes are not
    N, rows = 8, 1 << 25
    splits = [[[rows] for _ in range(N)] for _ in range(N)]
    send, recv = _ptrs(N, step=1 << 41), _ptrs(N, step=1 << 41, base=FAKE + (1 << 45))
    assert _status(gc.gc_all_to_all, send, recv, splits, 4096, stream=0) == gc.GC_ERR_UNSUPPORTED
    with pytest.raises(gc.GcError):
        gc.gc_bucket_plan_create([8, big], "bf16", gc.SIZE_MAX)   # one bucket of 2^40 + 32 bytes


def test_rank_buffers_layout():
    # host tensors stand in for device memory: only the offsets are checked
    bufs = gc.gc_rank_buffers(8, 1000, "bf16", device="cpu", stagger_bytes=4096, slot_align=1 << 20)
    base = bufs[0].data_ptr()
    for r, b in enumerate(bufs):
        assert b.numel() == 1000 and b.is_contiguous()
        assert b.data_ptr() - base == r * ((1 << 20) + 4096)
    with pytest.raises(ValueError):
        gc.gc_rank_buffers(2, 10, "fp32", device="cpu", stagger_bytes=6)


def test_bucket_all_reduce_validation():
    plan = gc.BucketPlan([8, 8], "bf16", 1 << 20)
    tensors = _ptrs(4)
    assert _status(gc.gc_bucket_all_reduce, plan.handle, 3, tensors, 2, stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(gc.gc_bucket_all_reduce, plan.handle, 0, tensors[:3] + [0], 2, stream=0) == gc.GC_ERR_INVALID_ARG
    overl = [tensors[0], tensors[0] + 8, tensors[2], tensors[3]]          # rank 0's two tensors overlap
    assert _status(gc.gc_bucket_all_reduce, plan.handle, 0, overl, 2, stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(gc.gc_bucket_all_reduce, plan.handle, 0, tensors, 2, sumsq=FAKE + 4,
                   stream=0) == gc.GC_ERR_INVALID_ARG                     # misaligned accumulator
    ip = gc.BucketPlan([8], "int32", 1 << 20)
    assert _status(gc.gc_bucket_all_reduce, ip.handle, 0, _ptrs(2), 2, op="avg", stream=0) == gc.GC_ERR_UNSUPPORTED
    assert _status(gc.gc_bucket_all_reduce, ip.handle, 0, _ptrs(2), 2, op="sum", sumsq=FAKE,
                   stream=0) == gc.GC_ERR_UNSUPPORTED
    assert _status(gc.gc_bucket_all_reduce, plan.handle, 0, tensors, 65, stream=0) == gc.GC_ERR_UNSUPPORTED


def test_moe_route_validation():
    route = gc.gc_moe_route
    nt = [100, 0, 37]
    need = gc.gc_moe_route_scratch_bytes(nt, 2, 4)
    # tiles of 1024 routes: 1 + 0 + 1 tiles x 12 experts, then 3 x 12 offsets, each 256-aligned
    assert need == 256 + 256
    assert gc.gc_moe_route_scratch_bytes(nt, 9, 4) == 0                     # topk > 8
    assert gc.gc_moe_route_scratch_bytes([1] * 64, 1, 129) == 0              # 64 * 129 experts > 8192
    assert gc.gc_moe_route_scratch_bytes([-1, 2, 3], 1, 1) == 0
    big = gc.gc_moe_route_scratch_bytes([10_000] * 2, 1, 4096)               # tiles of 8192 routes
    assert big == 4 * 8192 * 4 + 2 * 8192 * 4                             # 2 tiles per source
    ex, de = _ptrs(3), _ptrs(3, base=FAKE + (1 << 40))
    sp, sc = FAKE + (1 << 41), FAKE + (1 << 42)
    ok = dict(experts=ex, ntokens=nt, topk=2, experts_per_rank=4, splits=sp, dest=de, scratch=sc,
              scratch_bytes=need, stream=0)
    def st(**kw):
        a = dict(ok)
        a.update(kw)
        return _status(route, **a)
    assert st(scratch_bytes=need - 1) == gc.GC_ERR_INVALID_ARG
    assert st(scratch=sc + 16) == gc.GC_ERR_INVALID_ARG                     # not 256-aligned
    assert st(splits=sp + 4) == gc.GC_ERR_INVALID_ARG
    assert st(dest=de[:2] + [de[2] + 4]) == gc.GC_ERR_INVALID_ARG           # dest must be 8-aligned
    assert st(experts=[ex[0], ex[1], 0]) == gc.GC_ERR_INVALID_ARG           # null with tokens
    assert st(topk=0) == gc.GC_ERR_INVALID_ARG
    assert st(topk=9) == gc.GC_ERR_UNSUPPORTED
    assert st(scratch=de[0] + 512) == gc.GC_ERR_INVALID_ARG                 # scratch overlaps a dest table
    assert st(splits=ex[2]) == gc.GC_ERR_INVALID_ARG                        # an output over an input
    assert st(ntokens=[100, -1, 37]) == gc.GC_ERR_INVALID_ARG
    assert st(ntokens=[1 << 30, 1 << 30, 0]) == gc.GC_ERR_UNSUPPORTED       # 2^31 routes


def test_moe_route_noalloc_validation():
    # the variant without scratch: same checks, all made on the host before its scratch is looked up
    route = gc.gc_moe_route_noalloc
    nt = [100, 0, 37]
    ex, de = _ptrs(3), _ptrs(3, base=FAKE + (1 << 40))
    sp = FAKE + (1 << 41)
    ok = dict(experts=ex, ntokens=nt, topk=2, experts_per_rank=4, splits=sp, dest=de, stream=0)

    def st(**kw):
        a = dict(ok)
        a.update(kw)
        return _status(route, **a)
    big = [300_000] * 8                                                  # 38 MB of plan scratch
    assert gc.gc_moe_route_scratch_bytes(big, 8, 64) > gc.GC_MOE_ROUTE_NOALLOC_SCRATCH_BYTES
    assert st(experts=_ptrs(8), ntokens=big, topk=8, experts_per_rank=64,
              dest=_ptrs(8, base=FAKE + (1 << 40))) == gc.GC_ERR_UNSUPPORTED
    with pytest.raises(gc.GcError, match="needs .* bytes of scratch"):          # the refusal says why
        route(_ptrs(8), big, 8, 64, sp, _ptrs(8, base=FAKE + (1 << 40)), stream=0)
    assert st(splits=sp + 4) == gc.GC_ERR_INVALID_ARG
    assert st(dest=de[:2] + [de[2] + 4]) == gc.GC_ERR_INVALID_ARG
    assert st(experts=[ex[0], ex[1], 0]) == gc.GC_ERR_INVALID_ARG
    assert st(topk=0) == gc.GC_ERR_INVALID_ARG
    assert st(topk=9) == gc.GC_ERR_UNSUPPORTED
    assert st(splits=ex[2]) == gc.GC_ERR_INVALID_ARG
    assert st(dest=[de[0], de[1], de[0] + 64]) == gc.GC_ERR_INVALID_ARG   # two dest tables overlap


def test_moe_dispatch_combine_validation():
    nt, rows = [10, 0, 3], [8, 20, 0]
    tok, de = _ptrs(3), _ptrs(3, base=FAKE + (1 << 40))
    rv, w = _ptrs(3, base=FAKE + (1 << 41)), _ptrs(3, base=FAKE + (1 << 42))
    disp = dict(tokens=tok, ntokens=nt, dest=de, topk=2, row_bytes=64, recv=rv, recv_rows=rows, stream=0)
    def sd(**kw):
        a = dict(disp)
        a.update(kw)
        return _status(gc.gc_moe_dispatch, **a)
    assert sd(row_bytes=0) == gc.GC_ERR_INVALID_ARG
    assert sd(topk=9) == gc.GC_ERR_UNSUPPORTED
    assert sd(recv=[rv[0], rv[0] + 64, rv[2]]) == gc.GC_ERR_INVALID_ARG     # receive buffers overlap
    assert sd(recv=[tok[0] + 64] + rv[1:]) == gc.GC_ERR_INVALID_ARG         # receive over the tokens
    assert sd(recv=[de[0]] + rv[1:]) == gc.GC_ERR_INVALID_ARG               # receive over a dest table
    assert sd(dest=[de[0] + 4] + de[1:]) == gc.GC_ERR_INVALID_ARG
    assert sd(recv=[rv[0], 0, rv[2]]) == gc.GC_ERR_INVALID_ARG              # null with rows
    assert sd(recv_rows=[8, -1, 0]) == gc.GC_ERR_INVALID_ARG
    assert sd(ntokens=[0, 0, 0], recv_rows=[0, 0, 0]) == gc.GC_OK          # nothing to do
    comb = dict(expert_out=rv, expert_rows=rows, dest=de, weights=w, ntokens=nt, topk=2, hidden=32,
                dtype="bf16", out=tok, stream=0)
    def sc(**kw):
        a = dict(comb)
        a.update(kw)
        return _status(gc.gc_moe_combine, **a)
    assert sc(dtype="int32") == gc.GC_ERR_UNSUPPORTED
    assert sc(dtype=7) == gc.GC_ERR_INVALID_ARG
    assert sc(hidden=0) == gc.GC_ERR_INVALID_ARG
    assert sc(weights=None) == gc.GC_ERR_INVALID_ARG
    assert sc(weights=[w[0] + 2] + w[1:]) == gc.GC_ERR_INVALID_ARG          # misaligned weights
    assert sc(out=[tok[0], tok[1], tok[0] + 128]) == gc.GC_ERR_INVALID_ARG  # 10 rows of 64 B overlap
    assert sc(out=[w[0]] + tok[1:]) == gc.GC_ERR_INVALID_ARG                # output over the weights
    assert sc(out=[rv[1] + 64] + tok[1:]) == gc.GC_ERR_INVALID_ARG          # output over expert rows
    assert sc(dtype="fp32", out=[tok[0] + 2] + tok[1:]) == gc.GC_ERR_INVALID_ARG
    assert sc(ntokens=[0, 0, 0]) == gc.GC_OK


def test_fsdp2_validation():
    rs, ag = gc.gc_fsdp2_reduce_scatter, gc.gc_fsdp2_all_gather
    N, rows, cols = 4, [3, 2], [5, 2]                   # shards of rows: [1,1,1,0] and [1,1,0,0]
    G_ = [[FAKE + (r * 2 + p) * (1 << 30) for p in range(2)] for r in range(N)]
    S_ = [[FAKE + (1 << 40) + (r * 2 + p) * (1 << 30) for p in range(2)] for r in range(N)]
    kw = dict(rows=rows, cols=cols, nranks=N, in_dtype="bf16", out_dtype="fp32", op="avg", stream=0)
    assert _status(rs, G_, S_, **dict(kw, in_dtype="int32", out_dtype="int32")) == gc.GC_ERR_UNSUPPORTED
    assert _status(rs, G_, S_, **dict(kw, in_dtype="int32")) == gc.GC_ERR_UNSUPPORTED
    assert _status(rs, G_, S_, **dict(kw, order=5)) == gc.GC_ERR_INVALID_ARG
    bad = [row[:] for row in G_]
    bad[1][0] = 0
    assert _status(rs, bad, S_, **kw) == gc.GC_ERR_INVALID_ARG                 # a null gradient
    bad = [row[:] for row in S_]
    bad[0][1] = 0
    assert _status(rs, G_, bad, **kw) == gc.GC_ERR_INVALID_ARG                 # a null non-empty shard
    bad = [row[:] for row in S_]
    bad[2][1] = bad[3][1] = 0                                                  # empty shards may be null ...
    bad[0][0] = S_[1][0] + 8                                                   # ... but shards may not overlap
    assert _status(rs, G_, bad, **kw) == gc.GC_ERR_INVALID_ARG
    bad = [row[:] for row in S_]
    bad[0][0] = G_[1][0]                                                       # a shard over another rank's gradient
    assert _status(rs, G_, bad, **kw) == gc.GC_ERR_INVALID_ARG
    bad = [row[:] for row in S_]
    bad[1][0] = G_[1][0] + 2                                                   # not the in-place offset (5 elements)
    assert _status(rs, G_, bad, **dict(kw, out_dtype="bf16")) == gc.GC_ERR_INVALID_ARG
    bad = [row[:] for row in S_]
    bad[1][0] = S_[1][0] + 2                                                   # misaligned fp32 shard
    assert _status(rs, G_, bad, **kw) == gc.GC_ERR_INVALID_ARG
    assert _status(rs, G_, S_, rows=[0, 3], cols=[7, 0], nranks=N, in_dtype="bf16", stream=0) == gc.GC_OK
    # all-gather: params may not overlap each other or a shard, except the in-place slot
    P_ = [[FAKE + (1 << 41) + (r * 2 + p) * (1 << 30) for p in range(2)] for r in range(N)]
    akw = dict(rows=rows, cols=cols, nranks=N, dtype="bf16", stream=0)
    bad = [row[:] for row in P_]
    bad[3][1] = P_[2][1] + 4
    assert _status(ag, S_, bad, **akw) == gc.GC_ERR_INVALID_ARG
    bad = [row[:] for row in S_]
    bad[2][0] = P_[1][0]
    assert _status(ag, bad, P_, **akw) == gc.GC_ERR_INVALID_ARG
    assert _status(ag, S_, P_, **dict(akw, dtype=9)) == gc.GC_ERR_INVALID_ARG


def test_wire_order_validated_like_the_others_for_buckets():
    # the bf16 wire order is accepted by the bucket all-reduce; its arguments are checked as usual
    plan = gc.BucketPlan([8, 8], "bf16", 1 << 20)
    try:
        ptrs = _ptrs(4)
        assert _status(gc.gc_bucket_all_reduce, plan.handle, 0, ptrs[:3] + [0], 2, order="ring_wire",
                       stream=0) == gc.GC_ERR_INVALID_ARG
        assert _status(gc.gc_bucket_all_reduce, plan.handle, 0, ptrs, 2, order=7, stream=0) == gc.GC_ERR_INVALID_ARG
    finally:
        plan.close()


def test_hier_and_hsdp_validation():
    har, hrs = gc.gc_hier_all_reduce, gc.gc_hsdp_reduce_scatter
    s, r = _ptrs(8), _ptrs(8, base=FAKE + (1 << 40))
    assert _status(har, s, r, 4, count=0, dtype="bf16", stream=0) == gc.GC_OK
    assert _status(har, s, r, 3, count=16, dtype="bf16", stream=0) == gc.GC_ERR_INVALID_ARG     # 3 does not divide 8
    assert _status(har, s, r, 0, count=16, dtype="bf16", stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(har, s, r, 3, count=16, dtype="bf16", order="ring_wire", stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(har, s, r, 4, count=0, dtype="bf16", order="ring_wire", stream=0) == gc.GC_OK
    assert _status(har, s, r, 4, count=16, dtype="int32", op="avg", stream=0) == gc.GC_ERR_UNSUPPORTED
    assert _status(har, s, r[:7] + [r[6] + 8], 4, count=16, dtype="fp32", stream=0) == gc.GC_ERR_INVALID_ARG
    assert _status(har, s, r[:7] + [s[3] + 4], 4, count=16, dtype="fp32", stream=0) == gc.GC_ERR_INVALID_ARG
    kw = dict(recv_count=10, in_dtype="bf16", out_dtype="fp32", stream=0)
    assert _status(hrs, s, r, 4, **dict(kw, in_dtype="int32")) == gc.GC_ERR_UNSUPPORTED
    assert _status(hrs, s, r, 5, **kw) == gc.GC_ERR_INVALID_ARG
    assert _status(hrs, s, r[:7] + [r[7] + 2], 4, **kw) == gc.GC_ERR_INVALID_ARG                 # misaligned fp32
    # in place only at member i's chunk of the same rank, and only when the types match
    bad = r[:5] + [s[5] + 1 * 10 * 2] + r[6:]                                                   # rank 5 = member 1
    assert _status(hrs, s, bad, 4, **kw) == gc.GC_ERR_INVALID_ARG                              # bf16 -> fp32
    bad = r[:5] + [s[5] + 2 * 10 * 2] + r[6:]                                                   # member 2's chunk
    assert _status(hrs, s, bad, 4, **dict(kw, out_dtype="bf16")) == gc.GC_ERR_INVALID_ARG
    assert _status(hrs, s, r, 4, **dict(kw, recv_count=0)) == gc.GC_OK


class _DevTensor:
    """Stands in for a device tensor in the binding's checks: an address, a size
    and a layout flag.  Never dereferenced: every call below is stopped by the
    binding or by the library's host-side validation."""

    is_cuda = True

    def __init__(self, addr, nbytes, contiguous=True):
        self._addr, self._n, self._c = addr, nbytes, contiguous

    def numel(self):
        return self._n

    def element_size(self):
        return 1

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        return self._addr


def test_binding_rejects_short_strided_and_host_tensors():
    import torch
    T = _DevTensor
    send = [T(FAKE + i * (1 << 30), 64) for i in range(4)]
    recv = [T(FAKE + (1 << 40) + i * (1 << 30), 64) for i in range(4)]
    with pytest.raises(ValueError, match="buffers, the call needs 4"):      # recv list shorter than send
        gc.gc_all_reduce(send, recv[:3], count=16, dtype="fp32", stream=0)
    with pytest.raises(ValueError, match=r"recv\[2\]: 60 bytes"):           # one output too small
        gc.gc_all_reduce(send, recv[:2] + [T(recv[2].data_ptr(), 60)] + recv[3:], count=16, dtype="fp32", stream=0)
    with pytest.raises(ValueError, match="not contiguous"):
        gc.gc_all_reduce([T(FAKE, 64, contiguous=False)] + send[1:], recv, count=16, dtype="fp32", stream=0)
    with pytest.raises(ValueError, match="device"):                          # a host tensor
        gc.gc_all_reduce([torch.zeros(16)] + send[1:], recv, count=16, dtype="fp32", stream=0)
    # right sizes pass the binding; the library then rejects the partial overlap on the host
    bad = recv[:3] + [T(send[0].data_ptr() + 4, 64)]
    assert _status(gc.gc_all_reduce, send, bad, count=16, dtype="fp32", stream=0) == gc.GC_ERR_INVALID_ARG
    # reduce-scatter: send holds N * recv_count elements, recv recv_count of the output type
    with pytest.raises(ValueError, match=r"send\[0\]: 64 bytes, the call touches 72"):
        gc.gc_reduce_scatter(send, recv, recv_count=9, in_dtype="bf16", out_dtype="fp32", stream=0)
    with pytest.raises(ValueError, match=r"recv\[0\]"):
        gc.gc_all_gather(send, [T(FAKE + (1 << 40), 255)] + recv[1:], count=16, dtype="fp32", stream=0)
    # all-to-all: send[s] needs its rows to every destination, recv[d] the rows from every source
    sp = [[[1], [2]], [[3], [4]]]
    big = [T(FAKE + i * (1 << 30), 256) for i in range(2)]
    with pytest.raises(ValueError, match=r"recv\[1\]: 64 bytes"):           # 2 + 4 rows of 16 B
        gc.gc_all_to_all(big, recv[:2], sp, 16, stream=0)
    with pytest.raises(ValueError, match=r"send\[1\]: 64 bytes"):           # 3 + 4 rows of 16 B
        gc.gc_all_to_all(send[:2], big, sp, 16, stream=0)
    # MoE combine: out[s] holds ntokens[s] rows of hidden elements
    with pytest.raises(ValueError, match=r"out\[0\]"):
        gc.gc_moe_combine(recv[:2], [2, 2], send[:2], send[2:], [3, 0], 2, 16, "bf16", recv[2:], stream=0)
    with pytest.raises(ValueError, match="the call needs 2"):
        gc.gc_moe_dispatch(send[:2], [1, 1], send[2:3], 2, 16, recv[:2], [1, 1], stream=0)


def test_bucket_plan_checks_sizes_against_the_plan():
    T = _DevTensor
    plan = gc.BucketPlan([8, 8, 100], "bf16", 32, reverse=False)   # buckets [0, 1] and [2]
    try:
        assert plan.nbuckets == 2
        tensors = [T(FAKE + i * (1 << 30), n * 2) for i, n in enumerate([8, 8, 100] * 2)]
        bufs = [T(FAKE + (1 << 40) + r * (1 << 30), 32) for r in range(2)]
        short = list(tensors)
        short[4] = T(tensors[4].data_ptr(), 15)                    # rank 1, tensor 1: 16 B needed
        with pytest.raises(ValueError, match=r"tensors\[4\]: 15 bytes"):
            plan.pack(0, short, bufs, 2, stream=0)
        with pytest.raises(ValueError, match=r"tensors\[4\]"):
            plan.all_reduce(0, short, 2, stream=0)
        short[4] = None                                            # outside bucket 1: not checked
        with pytest.raises(ValueError, match=r"bucket_bufs\[0\]: 32 bytes"):
            plan.unpack(1, bufs, short, 2, stream=0)               # bucket 1 holds 100 bf16
        with pytest.raises(ValueError, match="the call needs 6"):
            plan.all_reduce(0, tensors[:5], 2, stream=0)
        with pytest.raises(ValueError, match="sumsq: 4 bytes"):
            plan.all_reduce(0, tensors, 2, sumsq=T(FAKE + (1 << 42), 4), stream=0)
    finally:
        plan.close()


def test_fsdp2_binding_checks_shard_sizes():
    T = _DevTensor
    N, rows, cols = 4, [3, 2], [5, 2]                   # shards of rows: [1,1,1,0] and [1,1,0,0]
    G_ = [[T(FAKE + (r * 2 + p) * (1 << 30), rows[p] * cols[p] * 2) for p in range(2)] for r in range(N)]
    S_ = [[T(FAKE + (1 << 40) + (r * 2 + p) * (1 << 30), 64) for p in range(2)] for r in range(N)]
    S_[2][1] = S_[3][1] = 0                              # empty shards may be NULL
    S_[1][0] = T(S_[1][0].data_ptr(), 5 * 4 - 1)         # one row of 5 fp32 needs 20 B
    with pytest.raises(ValueError, match=r"shards\[2\]: 19 bytes"):
        gc.gc_fsdp2_reduce_scatter(G_, S_, rows, cols, N, "bf16", "fp32", stream=0)
    S_[1][0] = T(S_[1][0].data_ptr(), 20)
    P_ = [[T(FAKE + (1 << 41) + (r * 2 + p) * (1 << 30), rows[p] * cols[p] * 2) for p in range(2)]
          for r in range(N)]
    P_[3][0] = T(P_[3][0].data_ptr(), 29)                # 3 x 5 bf16 = 30 B
    with pytest.raises(ValueError, match=r"params\[6\]: 29 bytes"):
        gc.gc_fsdp2_all_gather(S_, P_, rows, cols, N, "bf16", stream=0)


def test_binding_shard_extents_follow_the_shard_rule():
    """The binding sizes its FSDP2 checks with the dim-0 shard rule; it must
    agree with the oracle's (torch.chunk) rule for every shape, or a short
    shard could pass the check."""
    import random
    rng = random.Random(3)
    for _ in range(300):
        N = rng.randint(1, 64)
        P = rng.randint(1, 6)
        rows = [rng.choice([0, 1, rng.randint(0, 3 * N), rng.randint(0, 5000)]) for _ in range(P)]
        cols = [rng.randint(0, 9) for _ in range(P)]
        es = rng.choice([2, 4])
        got = gc._shard_bytes(rows, cols, N, es)
        want = [(hi - lo) * cols[p] * es for r in range(N)
                for p in range(P) for lo, hi in [OB.uneven_dim0_shards(rows[p], N)[r]]]
        assert got == want, (N, rows, cols)


@pytest.mark.parametrize("reverse", [True, False])
def test_bucket_tensors_keep_the_visiting_order_with_empty_tensors(reverse):
    import random
    rng = random.Random(7 if reverse else 8)
    for _ in range(50):
        numels = [rng.choice([0, 0, 1, rng.randint(0, 5000)]) for _ in range(rng.randint(1, 25))]
        cap = rng.randint(1, 20000)
        plan = gc.BucketPlan(numels, "bf16", cap, reverse=reverse)
        try:
            got = [plan.bucket_tensors(b) for b in range(plan.nbuckets)]
        finally:
            plan.close()
        assert got == OB.assign_buckets(numels, 2, cap, reverse=reverse), (numels, cap)


def test_rank_arena_layout():
    """Every rank owns one region; a buffer sits at the same offset of every
    region (256-byte steps), regions are region + stagger bytes apart, and a
    full region raises instead of spilling into the next rank's."""
    import torch
    arena = gc.RankArena(4, region_bytes=1 << 16, stagger_bytes=4096, device="cpu")
    a = arena.alloc(1000, "bf16")                    # 2000 B -> next offset 2048
    b = arena.alloc(10, "fp32")
    base = arena.slab.data_ptr()
    step = (1 << 16) + 4096
    for r in range(4):
        assert a[r].numel() == 1000 and a[r].dtype == torch.bfloat16 and a[r].is_contiguous()
        assert a[r].data_ptr() - base == r * step
        assert b[r].data_ptr() - base == r * step + 2048
    with pytest.raises(MemoryError):
        arena.alloc((1 << 16) // 4, "fp32")          # 64 KiB more does not fit the 62 KiB left
