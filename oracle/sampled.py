"""Single-element evaluation of the collectives (test infrastructure only).

At full workload sizes the step-by-step emulation in `collectives` does not fit
in host memory, but every output element of a reduction depends only on the N
inputs at one position, and every output row of a permutation comes from one
input row.  These functions evaluate chosen output positions directly from the
fold order the ring induces (DTLM §2 "Reduce-Scatter": chunk j is folded
starting at rank j+1 and ends at its owner j), and the tests pin them to the
step-by-step emulation on sizes where both run.
"""

import numpy as np

from .collectives import _epilogue, _widen, a2a_recv_offsets, a2a_send_offsets
from .numerics import bf16_to_f32, f32_to_bf16


def fold_start(positions, S, N, order, chunk=None):
    """First rank of the fold for each element position (ring: owner + 1; rank: 0)."""
    positions = np.asarray(positions, dtype=np.int64)
    if order == "rank":
        return np.zeros(positions.shape, dtype=np.int64)
    c = chunk if chunk is not None else (-(-S // N) if S else 1)
    owner = positions // c
    return (owner + 1) % N


def reduce_positions(values, dtype, starts, op, out_dtype, wire=None):
    """values[i][k] = rank i's input at the k-th sampled position; fold in the given rank order.

    Element k is folded as values[start_k], values[start_k + 1], ... (mod N),
    starting from the first term, then averaged and cast like the owner does.
    wire="bf16": each partial is rounded to bf16 before the next term is added
    (the ring's messages in the wire type).
    """
    values = np.asarray(values)
    N, m = values.shape
    wide = np.stack([_widen(values[i], dtype) for i in range(N)])
    cols = np.arange(m)
    starts = np.asarray(starts, dtype=np.int64)
    acc = wide[starts % N, cols].copy()
    with np.errstate(over="ignore", invalid="ignore"):
        for t in range(1, N):
            if wire == "bf16":
                acc = bf16_to_f32(f32_to_bf16(acc))
            acc = acc + wide[(starts + t) % N, cols]
    return _epilogue(acc, op, N, out_dtype)


def all_reduce_at(values, positions, S, dtype, op, order):
    """All-reduce outputs at the sampled positions (same value on every rank)."""
    N = np.asarray(values).shape[0]
    wire = "bf16" if order == "ring_wire" and dtype == "bf16" else None
    return reduce_positions(values, dtype, fold_start(positions, S, N, order), op, dtype, wire)


def reduce_scatter_at(values, owner, out_pos, recv_count, in_dtype, out_dtype, op, order):
    """Reduce-scatter output recv[owner][out_pos]; values[i][k] = send[i][owner*recv_count + out_pos]."""
    N = np.asarray(values).shape[0]
    owner = np.asarray(owner, dtype=np.int64)
    starts = (owner + 1) % N if order != "rank" else np.zeros_like(owner)
    wire = "bf16" if order == "ring_wire" and in_dtype == "bf16" else None
    return reduce_positions(values, in_dtype, starts, op, out_dtype, wire)


def reduce_scatter_owner(chunks, owner, in_dtype, out_dtype, op, order, wire=None):
    """Owner j's whole reduce-scatter output from chunks[i] = rank i's chunk j (any length).

    Every element of chunk j has the same fold order, so the chunk is folded as
    whole vectors: ranks j+1, j+2, ..., N-1, 0, ..., j in ring order (DTLM §2
    "Reduce-Scatter"), 0, 1, ..., N-1 in rank order, starting from the first
    term; wire="bf16" rounds each forwarded partial to bf16 first (DTLM §11).
    Then the owner's epilogue.  This is how the full-size checks stream one
    owner at a time through memory the step-by-step emulation cannot hold.
    """
    N = len(chunks)
    first = (owner + 1) % N if order != "rank" else 0
    acc = _widen(chunks[first], in_dtype)
    with np.errstate(over="ignore", invalid="ignore"):
        for t in range(1, N):
            if wire == "bf16":
                acc = bf16_to_f32(f32_to_bf16(acc))
            acc = acc + _widen(chunks[(first + t) % N], in_dtype)
    return _epilogue(acc, op, N, out_dtype)


def a2a_source_rows(splits, d, recv_rows):
    """For rows of rank d's receive buffer, the (source rank, source row) they come from."""
    splits = np.asarray(splits, dtype=np.int64)
    N, _, E = splits.shape
    soff = a2a_send_offsets(splits)
    roff = a2a_recv_offsets(splits)
    out_s = np.empty(len(recv_rows), dtype=np.int64)
    out_row = np.empty(len(recv_rows), dtype=np.int64)
    for k, row in enumerate(np.asarray(recv_rows, dtype=np.int64)):
        found = False
        for e in range(E):
            for s in range(N):
                lo = roff[s, d, e]
                if lo <= row < lo + splits[s, d, e]:
                    out_s[k] = s
                    out_row[k] = soff[s, d, e] + (row - lo)
                    found = True
                    break
            if found:
                break
        if not found:
            raise IndexError("row beyond the receive buffer")
    return out_s, out_row


def hier_fold_starts(positions, count, S, R, order, chunk=None):
    """(first group, first member) of the two-level fold of each element position.

    Element E lies in chunk i of the S chunks of length c1 = ceil(count / S)
    (or `chunk`) and in piece h of that chunk's R pieces of ceil(len_i / R);
    the ring folds groups from h + 1 and members from i + 1 (rank order: 0, 0).
    """
    positions = np.asarray(positions, dtype=np.int64)
    if order == "rank":
        z = np.zeros(positions.shape, dtype=np.int64)
        return z, z
    c1 = chunk if chunk is not None else (-(-count // S) if count else 1)
    i = positions // c1
    lo = np.minimum(count, i * c1)
    L = np.minimum(count, lo + c1) - lo
    c2 = np.maximum(1, -(-L // R))
    h = (positions - lo) // c2
    return (h + 1) % R, (i + 1) % S


def hier_reduce_block(values, S, g0, m0, dtype, op, out_dtype, wire=None):
    """hier_reduce_positions for a block of positions that share one fold start
    (a cell: one chunk i and one of its cross-group pieces h), folded as whole
    vectors: groups g0, g0+1, ... (mod R), inside each group members m0, m0+1,
    ... (mod S).  values[r] = rank r's inputs over the block.  wire="bf16"
    rounds every forwarded partial to bf16 at both levels (DTLM §11)."""
    N = len(values)
    R = N // S
    total = None
    with np.errstate(over="ignore", invalid="ignore"):
        for q in range(R):
            g = (g0 + q) % R
            part = _widen(values[g * S + m0], dtype)
            for t in range(1, S):
                if wire == "bf16":
                    part = bf16_to_f32(f32_to_bf16(part))
                part = part + _widen(values[g * S + (m0 + t) % S], dtype)
            if total is None:
                total = part
            else:
                if wire == "bf16":
                    total = bf16_to_f32(f32_to_bf16(total))
                total = total + part
    return _epilogue(total, op, N, out_dtype)


def hier_reduce_positions(values, S, g0, m0, dtype, op, out_dtype):
    """values[r][k]: rank r's input at the k-th sampled position (rank r = g * S + i).
    Groups folded from g0, each group's members from m0, fp32 partials, one epilogue."""
    values = np.asarray(values)
    N, m = values.shape
    R = N // S
    wide = np.stack([_widen(values[r], dtype) for r in range(N)])
    cols = np.arange(m)
    g0 = np.asarray(g0, dtype=np.int64)
    m0 = np.asarray(m0, dtype=np.int64)
    total = None
    with np.errstate(over="ignore", invalid="ignore"):
        for q in range(R):
            g = (g0 + q) % R
            part = wide[g * S + m0, cols].copy()
            for t in range(1, S):
                part = part + wide[g * S + (m0 + t) % S, cols]
            total = part if total is None else total + part
    return _epilogue(total, op, N, out_dtype)
