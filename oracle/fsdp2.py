"""FSDP2 per-parameter Shard(0) collectives (test infrastructure only).

DTLM §4, "FSDP2: DTensor / DeviceMesh 版本的完整生命周期": FSDP2 keeps every
parameter as its own DTensor sharded along dim 0 over the mesh, instead of one
flat buffer per unit.  When the world size does not divide dim 0 the shards
follow torch.chunk: ceil(rows / N) rows per rank, trailing ranks shorter or
empty.  All-Gather reassembles each parameter from the shards by offset;
Reduce-Scatter leaves rank j its rows of the sum (or mean) of every rank's full
gradient of that parameter, so each gradient shard lines up with the
parameter shard.

Per parameter, the reduce-scatter is the ring reduce-scatter of
`collectives.ring_reduce_scatter_partials` over the parameter's row shards as
chunks (chunk j folded from rank j+1 around to j), followed by the same owner
epilogue as the flat collectives; the all-gather is the ring all-gather of the
shards, any lengths.
"""

import numpy as np

from .buckets import uneven_dim0_shards
from .collectives import (_check_types, _epilogue, _ring_wire, rank_order_fold, ring_all_gather,
                          ring_reduce_scatter_partials, storage_dtype)


def shard_elems(rows, cols, nranks):
    """Element range [lo, hi) of each rank's dim-0 shard of a rows x cols parameter."""
    return [(lo * cols, hi * cols) for lo, hi in uneven_dim0_shards(rows, nranks)]


def reduce_scatter(grads, rows, cols, in_dtype, out_dtype=None, op="sum", order="ring"):
    """grads[r][p]: rank r's full gradient of parameter p (flat, rows[p] * cols[p]).
    Returns out[j][p], rank j's shard of parameter p's reduced gradient."""
    out_dtype = out_dtype or in_dtype
    _check_types(in_dtype, out_dtype, op)
    N = len(grads)
    P = len(rows)
    out = [[None] * P for _ in range(N)]
    for p in range(P):
        xs = [np.asarray(grads[r][p]).reshape(-1) for r in range(N)]
        chunks = shard_elems(rows[p], cols[p], N)
        ring, wire = _ring_wire(order, in_dtype)
        if ring:
            ys = ring_reduce_scatter_partials(xs, in_dtype, chunks, wire=wire)
        else:
            full = rank_order_fold(xs, in_dtype)
            ys = [full[lo:hi] for lo, hi in chunks]
        for j in range(N):
            out[j][p] = _epilogue(ys[j], op, N, out_dtype)
    return out


def all_gather(shards, rows, cols, dtype):
    """shards[r][p]: rank r's dim-0 shard of parameter p.  Returns full[d][p] for every rank d."""
    N = len(shards)
    P = len(rows)
    full = [[None] * P for _ in range(N)]
    for p in range(P):
        want = shard_elems(rows[p], cols[p], N)
        parts = []
        for r in range(N):
            x = np.asarray(shards[r][p], dtype=storage_dtype(dtype)).reshape(-1)
            if x.size != want[r][1] - want[r][0]:
                raise ValueError("shard size does not match the Shard(0) rule")
            parts.append(x)
        got = ring_all_gather(parts)
        for d in range(N):
            full[d][p] = got[d]
    return full
