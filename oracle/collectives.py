"""Collectives emulated on the CPU, step by step (test infrastructure only).

N "ranks" are N numpy arrays.  Supported element types, named as strings:
  "bf16"   uint16 bit patterns; widened to fp32 exactly, reduced in fp32
  "fp32"   float32; reduced in fp32
  "int32"  int32; reduced with wrap-around modulo 2**32

Definitions followed (DTLM §2 "通信操作"):
  * Reduce-Scatter.  Rank i's buffer G_i is cut into N chunks; x_{j,i} is the
    chunk j of G_i.  Rank j ends with y_j = sum over i of x_{j,i}.
  * All-Gather.  Rank i holds shard p_i; every rank ends with
    concat(p_0, ..., p_{N-1}).
  * All-Reduce = Reduce-Scatter followed by All-Gather; with averaging,
    G = sum_i G_i / N  (DTLM §2 "All-Reduce"; NXMR §2.1).
  * All-to-All.  Rank s sends a different block to every rank d, and rank d
    receives the blocks addressed to it from every rank (DTLM §2 "All-to-All";
    with irregular block sizes this is All-to-AllV, DTLM §8).

Ring schedule (DTLM §2 "Reduce-Scatter", the N = 4 worked example; NXMR §2.2):
data moves rank r -> rank r+1 (mod N).  Chunk j starts at rank j+1 and its last
hop lands on its owner j, so after N-1 steps rank j holds y_j.  At step s
(1 <= s <= N-1) rank r sends its partial of chunk (r - s) mod N; the receiver
adds its own contribution to that partial.  The fold order of chunk j is
therefore x_{j,j+1}, x_{j,j+2}, ..., x_{j,N-1}, x_{j,0}, ..., x_{j,j}, starting
from the first term itself (never from a zero).  The All-Gather ring moves
shard (r - s + 1) mod N from rank r to rank r+1 at step s, and each rank
finally orders what it holds by shard index (DTLM §2 "All-Reduce", the
All-Gather half of the N = 4 example).

Chunking.  The pages cut a buffer of D bytes into N chunks of about D/N
(DTLM §2).  When N does not divide the element count S, the reading taken is
the torch.chunk-like rule DTLM §4 (FSDP2, uneven Shard(0)) spells out: every
chunk holds c = ceil(S / N) elements except the trailing ones, which are short
or empty.

Averaging.  The owner divides its fp32 sum by N once, with one IEEE division,
and then casts to the output type (DTLM §2 "All-Reduce": G = sum_i G_i / N;
DTLM §4 FSDP1: division by world_size after the reduce).
"""

from dataclasses import dataclass, field
from fractions import Fraction

import numpy as np

from .numerics import bf16_to_f32, f32_to_bf16

DTYPES = ("bf16", "fp32", "int32")
_STORAGE = {"bf16": np.uint16, "fp32": np.float32, "int32": np.int32}
ELEM_BYTES = {"bf16": 2, "fp32": 4, "int32": 4}


def storage_dtype(dtype):
    return _STORAGE[dtype]


def _widen(x, dtype):
    """Element values in the reduction type (fp32 for floats, int32 for ints)."""
    x = np.asarray(x, dtype=_STORAGE[dtype])
    if dtype == "bf16":
        return bf16_to_f32(x)
    return x.copy()


def _epilogue(acc, op, nranks, out_dtype):
    with np.errstate(over="ignore", invalid="ignore"):
        return _epilogue_impl(acc, op, nranks, out_dtype)


def _epilogue_impl(acc, op, nranks, out_dtype):
    """Average (one fp32 division by N) if asked, then cast to the output type."""
    if op == "avg":
        if out_dtype == "int32" or acc.dtype != np.float32:
            raise ValueError("avg is defined for floating-point data only")
        acc = acc / np.float32(nranks)
    if out_dtype == "bf16":
        return f32_to_bf16(acc)
    if out_dtype == "fp32":
        if acc.dtype != np.float32:
            raise ValueError("int32 data cannot be cast to fp32 here")
        return acc.astype(np.float32)
    if acc.dtype != np.int32:
        raise ValueError("float data cannot be cast to int32 here")
    return acc.astype(np.int32)


def owner_chunks(S, N):
    """Chunk j = [j*c, min(S, (j+1)*c)) with c = ceil(S/N); trailing chunks may be short or empty."""
    if N < 1:
        raise ValueError("need at least one rank")
    c = -(-S // N) if S else 0
    out = []
    for j in range(N):
        lo = min(S, j * c)
        hi = min(S, (j + 1) * c)
        out.append((lo, hi))
    return out


@dataclass
class Message:
    step: int
    src: int
    dst: int
    chunk: int
    terms: tuple          # source ranks whose contributions the message carries
    elems: int


@dataclass
class RingTrace:
    """What the emulated ring did: every message, and per-rank sent elements."""
    nranks: int
    messages: list = field(default_factory=list)
    sent_elems: list = None
    steps: int = 0

    def __post_init__(self):
        if self.sent_elems is None:
            self.sent_elems = [0] * self.nranks


def _ieee(fn):
    """Run fn with numpy's overflow / invalid warnings off: inf and NaN results are intended IEEE behaviour."""
    def wrapped(*a, **k):
        with np.errstate(over="ignore", invalid="ignore"):
            return fn(*a, **k)
    wrapped.__doc__, wrapped.__name__ = fn.__doc__, fn.__name__
    return wrapped


def _on_wire(part, wire):
    """What a message carries: the partial rounded to the wire type (bf16), or unchanged."""
    if wire == "bf16":
        return bf16_to_f32(f32_to_bf16(part))
    return part


@_ieee
def ring_reduce_scatter_partials(xs, dtype, chunks=None, trace=None, wire=None):
    """Run the ring Reduce-Scatter and return y_j (in the reduction type) for every owner j.

    xs[i] is rank i's full buffer.  chunks[j] = (lo, hi) is chunk j's element
    range; by default owner_chunks(S, N).  wire="bf16": every message is the
    sender's partial rounded to bf16 (a ring that communicates in the
    gradient's type; DTLM §11 "精度和分布式通信的关系"), and the receiver adds
    its own contribution to that rounded value in fp32.
    """
    N = len(xs)
    S = len(xs[0])
    if any(len(x) != S for x in xs):
        raise ValueError("every rank must hold the same number of elements")
    if chunks is None:
        chunks = owner_chunks(S, N)
    wide = [_widen(x, dtype) for x in xs]

    def piece(rank, j):
        lo, hi = chunks[j]
        return wide[rank][lo:hi]

    if N == 1:
        return [piece(0, 0).copy()]

    # Before step 1, rank r's outgoing message is its own contribution to
    # chunk (r - 1) mod N.
    holding = {r: ((r - 1) % N, piece(r, (r - 1) % N).copy(), (r,)) for r in range(N)}
    for s in range(1, N):
        delivered = {}
        for r in range(N):
            k, part, terms = holding[r]
            q = (r + 1) % N
            if trace is not None:
                trace.messages.append(Message(s, r, q, k, terms, part.size))
                trace.sent_elems[r] += part.size
            delivered[q] = (k, _on_wire(part, wire) + piece(q, k), terms + (q,))
        holding = delivered
        if trace is not None:
            trace.steps += 1
    for j in range(N):
        assert holding[j][0] == j
    return [holding[j][1] for j in range(N)]


def ring_all_gather(shards, trace=None):
    """Ring All-Gather of per-rank shards (any lengths); every rank gets the concatenation."""
    N = len(shards)
    have = [{r: np.asarray(shards[r]).copy()} for r in range(N)]
    for s in range(1, N):
        in_flight = []
        for r in range(N):
            k = (r - s + 1) % N
            q = (r + 1) % N
            buf = have[r][k]
            in_flight.append((q, k, buf))
            if trace is not None:
                trace.messages.append(Message(s, r, q, k, (k,), buf.size))
                trace.sent_elems[r] += buf.size
        for q, k, buf in in_flight:
            assert k not in have[q]
            have[q][k] = buf.copy()
        if trace is not None:
            trace.steps += 1
    return [np.concatenate([have[r][k] for k in range(N)]) for r in range(N)]


def _check_types(in_dtype, out_dtype, op):
    if in_dtype not in DTYPES or out_dtype not in DTYPES:
        raise ValueError("unknown dtype")
    if (in_dtype == "int32") != (out_dtype == "int32"):
        raise ValueError("int32 reduces to int32 only")
    if op not in ("sum", "avg"):
        raise ValueError("op must be sum or avg")


@_ieee
def rank_order_fold(xs, dtype):
    """The direct N-way fold ((x_0 + x_1) + x_2) + ... + x_{N-1}, in the reduction type.

    This is the plain reading of the Reduce example "g0 + g1 + g2 + g3"
    (DTLM §2 "Reduce"); the pages give no other order for a non-ring sum.
    """
    acc = _widen(xs[0], dtype)
    for x in xs[1:]:
        acc = acc + _widen(x, dtype)
    return acc


def _ring_wire(order, in_dtype):
    """(is a ring order, wire type) for order in ring / ring_wire / rank."""
    if order not in ("ring", "ring_wire", "rank"):
        raise ValueError("order must be ring, ring_wire or rank")
    wire = in_dtype if order == "ring_wire" and in_dtype == "bf16" else None
    return order != "rank", wire


def reduce_scatter(xs, in_dtype, out_dtype=None, op="sum", order="ring", trace=None):
    """Reduce-Scatter with equal chunks: N must divide the per-rank count (the caller pads, as FSDP does).
    order "ring_wire" is the ring whose messages are rounded to the input type (bf16 only)."""
    out_dtype = out_dtype or in_dtype
    _check_types(in_dtype, out_dtype, op)
    N = len(xs)
    S = len(xs[0])
    if S % N:
        raise ValueError("reduce_scatter needs a per-rank count divisible by N")
    rc = S // N
    chunks = [(j * rc, (j + 1) * rc) for j in range(N)]
    ring, wire = _ring_wire(order, in_dtype)
    if ring:
        ys = ring_reduce_scatter_partials(xs, in_dtype, chunks, trace, wire)
    else:
        full = rank_order_fold(xs, in_dtype)
        ys = [full[lo:hi] for lo, hi in chunks]
    return [_epilogue(y, op, N, out_dtype) for y in ys]


def all_gather(shards, trace=None):
    """All-Gather: every rank receives concat(shard_0, ..., shard_{N-1})."""
    return ring_all_gather(shards, trace)


def all_reduce(xs, dtype, op="sum", order="ring", trace=None):
    """All-Reduce as ring Reduce-Scatter, owner epilogue, ring All-Gather.

    order="ring": chunks by owner_chunks (any S), fold order of the ring.
    order="ring_wire": the same ring, every message rounded to bf16 (bf16 data only).
    order="rank": every element folded in rank order 0..N-1 (no chunk dependence).
    """
    _check_types(dtype, dtype, op)
    N = len(xs)
    S = len(xs[0])
    chunks = owner_chunks(S, N)
    ring, wire = _ring_wire(order, dtype)
    if ring:
        ys = ring_reduce_scatter_partials(xs, dtype, chunks, trace, wire)
    else:
        full = rank_order_fold(xs, dtype)
        ys = [full[lo:hi] for lo, hi in chunks]
    shards = [_epilogue(y, op, N, dtype) for y in ys]
    return ring_all_gather(shards, trace)


def exact_sum(values):
    """Exact rational sum of a sequence of finite floats or ints (brute force)."""
    total = Fraction(0)
    for v in values:
        total += Fraction(float(v)) if isinstance(v, (float, np.floating)) else Fraction(int(v))
    return total


# ---------------------------------------------------------------- all-to-all

def a2a_send_offsets(splits):
    """Row offset of block (s, d, e) in rank s's send buffer, laid out by (d, e)."""
    splits = np.asarray(splits, dtype=np.int64)
    N, N2, E = splits.shape
    off = np.zeros_like(splits)
    for s in range(N):
        run = 0
        for d in range(N2):
            for e in range(E):
                off[s, d, e] = run
                run += splits[s, d, e]
    return off


def a2a_recv_offsets(splits):
    """Row offset of block (s, d, e) in rank d's receive buffer, laid out by (e, s)."""
    splits = np.asarray(splits, dtype=np.int64)
    N, N2, E = splits.shape
    off = np.zeros_like(splits)
    for d in range(N2):
        run = 0
        for e in range(E):
            for s in range(N):
                off[s, d, e] = run
                run += splits[s, d, e]
    return off


def all_to_all(sends, splits, row_elems):
    """All-to-AllV with an expert dimension: a pure block permutation of rows.

    sends[s] is rank s's send buffer: rows grouped by destination rank d, then
    by local expert e (splits[s][d][e] rows each).  Rank d receives, grouped by
    local expert e, then by source s, the block (s, d, e), rows in their sent
    order.  With one expert per rank this is plain All-to-AllV: rank d gets the
    blocks a_{0,d}, a_{1,d}, ... in source order (DTLM §2 "All-to-All").
    """
    splits = np.asarray(splits, dtype=np.int64)
    N, N2, E = splits.shape
    if N != N2:
        raise ValueError("splits must be [N][N][E]")
    for s in range(N):
        if len(sends[s]) != int(splits[s].sum()) * row_elems:
            raise ValueError("send buffer size does not match its splits")
    soff = a2a_send_offsets(splits)
    recvs = []
    for d in range(N):
        parts = []
        for e in range(E):
            for s in range(N):
                lo = int(soff[s, d, e]) * row_elems
                hi = lo + int(splits[s, d, e]) * row_elems
                parts.append(np.asarray(sends[s])[lo:hi])
        recvs.append(np.concatenate(parts) if parts else np.zeros(0, dtype=np.asarray(sends[0]).dtype))
    return recvs
