"""Hierarchical (two-level) all-reduce and the HSDP gradient reduce-scatter
(test infrastructure only).

AIG6 Table 6-2 lists the hierarchical all-reduce as two-level aggregation
matching the physical topology; AIG6 §6.3.6 describes HSDP on 2 nodes x 8
GPUs: parameters sharded across the 8 GPUs of a node and gathered within it,
gradients combined across the nodes; DTLM §4 (FSDP2, DeviceMesh) describes
HSDP as a 2-D mesh with one dimension that shards and one that replicates.

Mesh: N = R * S ranks in R groups of S (a group = a node = one shard group);
rank g * S + i is member i of group g.  The two-level all-reduce is the
composition of three rings, each emulated step by step by `collectives`:

  1. inside every group, a ring reduce-scatter over its S members: member i
     ends with chunk i of the group's sum (fp32 partials, no epilogue);
  2. across groups, for every i, a ring all-reduce of chunk i over the R
     members (g, i), g = 0..R-1, on those fp32 partials; the owner of each
     piece applies the epilogue once (avg: divide by N, then round to the
     output type);
  3. inside every group, a ring all-gather of the chunks.

The HSDP gradient reduce-scatter stops after step 2: rank (g, i) keeps chunk
i of the global reduction, the same on every group.  order="rank" replaces
each ring fold by the rank-order fold at its level.  order="ring_wire" is the
ring schedule whose every message is rounded to bf16 (bf16 data only; DTLM §11
"精度和分布式通信的关系": low-precision communication, fp32 arithmetic): inside
a group each forwarded partial is rounded before the next member adds its
term, and across groups each group's partial is rounded when it is sent on to
the next group.  For fp32 and int32 data the wire changes nothing.
"""

import numpy as np

from .collectives import (_check_types, _epilogue, owner_chunks, rank_order_fold, ring_all_gather,
                          ring_reduce_scatter_partials)


def _level_one(xs, S, dtype, chunks, order, wire):
    """Per group g, per member i: the group's partial sum of chunk i (reduction type)."""
    R = len(xs) // S
    parts = []
    for g in range(R):
        members = [xs[g * S + k] for k in range(S)]
        if order == "ring":
            parts.append(ring_reduce_scatter_partials(members, dtype, chunks, wire=wire))
        else:
            full = rank_order_fold(members, dtype)
            parts.append([full[lo:hi] for lo, hi in chunks])
    return parts


def _level_two(parts, i, acc_dtype, op, N, out_dtype, order, wire):
    """Chunk i reduced across the groups: the R pieces (one per owner group), after the epilogue."""
    R = len(parts)
    cross = [parts[g][i] for g in range(R)]
    L = len(cross[0])
    pieces = owner_chunks(L, R)
    if order == "ring":
        ys = ring_reduce_scatter_partials(cross, acc_dtype, pieces, wire=wire)
    else:
        full = rank_order_fold(cross, acc_dtype)
        ys = [full[lo:hi] for lo, hi in pieces]
    return [_epilogue(y, op, N, out_dtype) for y in ys]


def _check(xs, S, order, dtype):
    """(N, R, order of the folds, wire type) for a mesh of groups of S."""
    N = len(xs)
    if S < 1 or N % S:
        raise ValueError("the group size must divide the number of ranks")
    if order not in ("ring", "rank", "ring_wire"):
        raise ValueError("order must be ring, rank or ring_wire")
    wire = "bf16" if order == "ring_wire" and dtype == "bf16" else None
    return N, N // S, ("rank" if order == "rank" else "ring"), wire


def all_reduce(xs, S, dtype, op="sum", order="ring"):
    """Two-level all-reduce of N = R * S rank buffers (any length)."""
    _check_types(dtype, dtype, op)
    N, R, order, wire = _check(xs, S, order, dtype)
    count = len(xs[0])
    chunks = owner_chunks(count, S)
    acc = "int32" if dtype == "int32" else "fp32"
    parts = _level_one(xs, S, dtype, chunks, order, wire)
    shards = []
    for i in range(S):
        pieces = _level_two(parts, i, acc, op, N, dtype, order, wire)
        shards.append(ring_all_gather(pieces)[0])       # the cross-group all-gather of the pieces
    full = ring_all_gather(shards)                       # step 3, inside a group (every group alike)
    return [full[0].copy() for _ in range(N)]


def hsdp_reduce_scatter(xs, S, in_dtype, out_dtype=None, op="sum", order="ring"):
    """HSDP gradient sync: rank g * S + i receives chunk i of the reduction over all N
    ranks.  S must divide the per-rank count (the flat gradient is padded, as FSDP does)."""
    out_dtype = out_dtype or in_dtype
    _check_types(in_dtype, out_dtype, op)
    N, R, order, wire = _check(xs, S, order, in_dtype)
    count = len(xs[0])
    if count % S:
        raise ValueError("hsdp_reduce_scatter needs a per-rank count divisible by the group size")
    rc = count // S
    chunks = [(i * rc, (i + 1) * rc) for i in range(S)]
    acc = "int32" if in_dtype == "int32" else "fp32"
    parts = _level_one(xs, S, in_dtype, chunks, order, wire)
    out = [None] * N
    for i in range(S):
        shard = np.concatenate(_level_two(parts, i, acc, op, N, out_dtype, order, wire))
        for g in range(R):
            out[g * S + i] = shard.copy()
    return out
