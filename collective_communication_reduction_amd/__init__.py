"""Gradient-synchronisation collectives on one MI355X: Python binding of libgc.

A thin ctypes layer over the C ABI declared in include/gc.h.  It only marshals
arguments: it turns lists of tensors (or raw device addresses) into pointer
arrays, maps dtype/op/order names onto the C enums, passes torch's current HIP
stream, and raises GcError for a non-OK status.  Since the library sees only
addresses, a tensor is checked here first (a contiguous device tensor that
holds every byte the call touches, else ValueError); raw addresses and
gc_pointers arrays are the caller's responsibility.  Every collective runs in the
HIP kernels of libgc.so; there is no other implementation to fall back to, and
importing this package fails if the library has not been built
(python collective_communication_reduction_amd/build.py).

The functions carry the C names:
  gc_all_reduce, gc_reduce_scatter, gc_all_gather, gc_all_to_all,
  gc_all_reduce_scratch_bytes, gc_bucket_plan_create / _query / _destroy,
  gc_bucket_pack, gc_bucket_unpack, gc_bucket_all_reduce, gc_status_string,
  gc_version, gc_last_hip_error
plus BucketPlan, a small owner of a gc_bucket_plan handle; RankArena, which
gives each rank its own region of HBM; gc_rank_buffers, which lays N rank
buffers out in one allocation with a per-rank stagger; and gc_pointers, which
marshals a pointer array once for buffers synchronised every step.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgc.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python collective_communication_reduction_amd/build.py)")

# PyTorch ships its own HIP runtime, which its libraries request as
# "libamdhip64.so"; libgc requests "libamdhip64.so.7".  Importing torch first
# makes libgc bind to the runtime already in the process, so both sides share
# one runtime (and torch's streams and allocations are valid for libgc).
# Loading libgc first would pull in the system runtime as a second copy.
try:
    import torch  # noqa: F401
except ImportError:  # pragma: no cover - the library itself does not need torch
    torch = None

_lib = ctypes.CDLL(LIB_PATH)

GC_MAX_RANKS = 64
GC_OK, GC_ERR_INVALID_ARG, GC_ERR_UNSUPPORTED, GC_ERR_HIP, GC_ERR_NO_MEMORY = range(5)
GC_INT32, GC_FP32, GC_BF16 = 0, 1, 2
GC_SUM, GC_AVG = 0, 1
GC_ORDER_RING, GC_ORDER_RANK, GC_ORDER_RING_WIRE = 0, 1, 2
GC_AR_FUSED, GC_AR_RS_AG = 0, 1
SIZE_MAX = (1 << 64) - 1

_DTYPE = {"int32": GC_INT32, "fp32": GC_FP32, "bf16": GC_BF16}
_OP = {"sum": GC_SUM, "avg": GC_AVG}
_ORDER = {"ring": GC_ORDER_RING, "rank": GC_ORDER_RANK, "ring_wire": GC_ORDER_RING_WIRE}
_ALGO = {"fused": GC_AR_FUSED, "rs_ag": GC_AR_RS_AG}

_vp, _sz, _int = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_VPP = ctypes.POINTER(ctypes.c_void_p)


def _sig(name, restype, *argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_c_rs = _sig("gc_reduce_scatter", _int, _VPP, _VPP, _sz, _int, _int, _int, _int, _int, _vp)
_c_ag = _sig("gc_all_gather", _int, _VPP, _VPP, _sz, _int, _int, _vp)
_c_ar_scratch = _sig("gc_all_reduce_scratch_bytes", _sz, _sz, _int, _int, _int)
_c_ar = _sig("gc_all_reduce", _int, _VPP, _VPP, _sz, _int, _int, _int, _int, _int, _vp, _sz, _vp)
_c_a2a = _sig("gc_all_to_all", _int, _VPP, _VPP, ctypes.POINTER(ctypes.c_int64), _int, _int, _sz, _vp)
_I64P = ctypes.POINTER(ctypes.c_int64)
_SZP = ctypes.POINTER(ctypes.c_size_t)
_c_fsdp2_rs = _sig("gc_fsdp2_reduce_scatter", _int, _VPP, _VPP, _SZP, _SZP, _int, _int, _int, _int, _int, _int, _vp)
_c_hier_ar = _sig("gc_hier_all_reduce", _int, _VPP, _VPP, _sz, _int, _int, _int, _int, _int, _vp)
_c_hsdp_rs = _sig("gc_hsdp_reduce_scatter", _int, _VPP, _VPP, _sz, _int, _int, _int, _int, _int, _int, _vp)
_c_fsdp2_ag = _sig("gc_fsdp2_all_gather", _int, _VPP, _VPP, _SZP, _SZP, _int, _int, _int, _vp)
_c_moe_scratch = _sig("gc_moe_route_scratch_bytes", _sz, _I64P, _int, _int, _int)
_c_moe_route = _sig("gc_moe_route", _int, _VPP, _I64P, _int, _int, _int, _vp, _VPP, _vp, _sz, _vp)
_c_moe_route_noalloc = _sig("gc_moe_route_noalloc", _int, _VPP, _I64P, _int, _int, _int, _vp, _VPP, _vp)
_c_moe_dispatch = _sig("gc_moe_dispatch", _int, _VPP, _I64P, _VPP, _int, _int, _sz, _VPP, _I64P, _vp)
_c_moe_combine = _sig("gc_moe_combine", _int, _VPP, _I64P, _VPP, _VPP, _I64P, _int, _int, _sz, _int, _VPP, _vp)
_c_plan_create = _sig("gc_bucket_plan_create", _int, ctypes.POINTER(ctypes.c_size_t), _int, _int, _sz, _int, _sz,
                      ctypes.POINTER(_vp))
_c_plan_query = _sig("gc_bucket_plan_query", _int, _vp, ctypes.POINTER(_int), ctypes.POINTER(ctypes.c_size_t),
                     ctypes.POINTER(_int), ctypes.POINTER(ctypes.c_size_t))
_c_pack = _sig("gc_bucket_pack", _int, _vp, _int, _VPP, _VPP, _int, _vp)
_c_unpack = _sig("gc_bucket_unpack", _int, _vp, _int, _VPP, _VPP, _int, _vp)
_c_bucket_ar = _sig("gc_bucket_all_reduce", _int, _vp, _int, _VPP, _int, _int, _int, _vp, _vp)
_c_plan_destroy = _sig("gc_bucket_plan_destroy", None, _vp)
_c_status = _sig("gc_status_string", ctypes.c_char_p, _int)
_c_version = _sig("gc_version", _int)
_c_last_hip = _sig("gc_last_hip_error", _int)


class GcError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        detail = f" (hipError_t {gc_last_hip_error()})" if status == GC_ERR_HIP else ""
        super().__init__(f"{what}: {gc_status_string(status)}{detail}")


def gc_last_hip_error():
    """hipError_t of the last HIP call that failed inside libgc on this thread (0 if none)."""
    return _c_last_hip()


def gc_status_string(status):
    return _c_status(int(status)).decode()


def gc_version():
    return _c_version()


def _check(status, what):
    if status != GC_OK:
        raise GcError(status, what)


# ------------------------------------------------------------------ marshalling

_ES = {GC_INT32: 4, GC_FP32: 4, GC_BF16: 2}


def _buf(x, nbytes, what):
    """Address of one device buffer that a call reads or writes for nbytes bytes.

    A tensor must be a contiguous device tensor of at least nbytes bytes: the C
    ABI sees only its address, so a host, strided or short tensor would reach the
    kernels as an out-of-bounds access.  A raw integer address (or None) is the
    caller's responsibility and passes unchecked."""
    if x is None or isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError(f"{what}: a device (cuda) tensor is required")
    if not x.is_contiguous():
        raise ValueError(f"{what}: the tensor is not contiguous")
    have = x.numel() * x.element_size()
    if have < nbytes:
        raise ValueError(f"{what}: {have} bytes, the call touches {nbytes}")
    return x.data_ptr()


def _bufs(xs, n, nbytes, what):
    """Pointer array of the first n buffers of xs, each checked by _buf.

    nbytes is one size for every buffer or a sequence with one size per buffer.
    A pointer array made by gc_pointers passes unchecked but must hold n
    entries; None passes as NULL (the library rejects it)."""
    if xs is None:
        return None
    if len(xs) < n:
        raise ValueError(f"{what}: {len(xs)} buffers, the call needs {n}")
    if isinstance(xs, ctypes.Array):
        return xs
    arr = (ctypes.c_void_p * max(1, len(xs)))()
    for i, x in enumerate(xs):
        need = nbytes if isinstance(nbytes, int) else (int(nbytes[i]) if i < n else 0)
        arr[i] = _buf(x, need if i < n else 0, f"{what}[{i}]")
    return arr


def _dtype_code(x):
    if isinstance(x, str):
        return _DTYPE[x]
    if isinstance(x, int):
        return x
    import torch
    return {torch.bfloat16: GC_BF16, torch.float32: GC_FP32, torch.int32: GC_INT32}[x]


def _enum(table, x):
    return table[x] if isinstance(x, str) else int(x)


def gc_pointers(tensors):
    """Marshal a list of tensors (or addresses, or None) into a pointer array once.

    Every call that takes a list also accepts the returned array, which saves
    rebuilding it when the same buffers are synchronised every step (DDP's
    gradient tensors persist across steps).  Tensors must be contiguous device
    tensors; their sizes are not known here, so the calls that take the array
    trust it."""
    xs = list(tensors)
    return _bufs(xs, len(xs), 0, "gc_pointers")


def _stream(stream, like=None):
    """HIP stream handle: an explicit int / torch stream, else torch's current stream on like's device."""
    if stream is None:
        import torch
        dev = like.device if hasattr(like, "device") and like.device.type == "cuda" else None
        if dev is None and not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _first(xs):
    """First tensor-like element (its device picks the stream), or None."""
    if xs is None or isinstance(xs, ctypes.Array):
        return None
    for x in xs:
        if x is not None and not isinstance(x, int):
            return x
    return None


def _numel(xs, count):
    if count is not None:
        return int(count)
    return int(xs[0].numel())


def _infer_dtype(xs, dtype):
    if dtype is not None:
        return _dtype_code(dtype)
    return _dtype_code(xs[0].dtype)


# ------------------------------------------------------------------ collectives

def gc_all_reduce(send, recv=None, op="avg", order="ring", algo="fused", scratch=None, scratch_bytes=None,
                  count=None, dtype=None, stream=None):
    """All-reduce N rank buffers; recv defaults to send (in place).  See include/gc.h."""
    recv = send if recv is None else recv
    n = len(send)
    t = _infer_dtype(send, dtype)
    cnt = _numel(send, count)
    a = _enum(_ALGO, algo)
    if scratch_bytes is None:
        scratch_bytes = scratch.numel() * scratch.element_size() if hasattr(scratch, "numel") else 0
    nb = cnt * _ES.get(t, 0)
    _check(_c_ar(_bufs(send, n, nb, "send"), _bufs(recv, n, nb, "recv"), cnt, n, t, _enum(_OP, op),
                 _enum(_ORDER, order), a, _buf(scratch, int(scratch_bytes), "scratch"), int(scratch_bytes),
                 _stream(stream, _first(send))), "gc_all_reduce")
    return recv


def gc_all_reduce_scratch_bytes(count, nranks, dtype, algo="rs_ag"):
    return int(_c_ar_scratch(int(count), int(nranks), _dtype_code(dtype), _enum(_ALGO, algo)))


def gc_reduce_scatter(send, recv, op="avg", order="ring", recv_count=None, in_dtype=None, out_dtype=None,
                      stream=None):
    """Reduce-scatter: recv[j] = op_i send[i][j*recv_count : (j+1)*recv_count]."""
    n = len(send)
    ti = _infer_dtype(send, in_dtype)
    to = _infer_dtype(recv, out_dtype)
    rc = _numel(recv, recv_count)
    _check(_c_rs(_bufs(send, n, n * rc * _ES.get(ti, 0), "send"), _bufs(recv, n, rc * _ES.get(to, 0), "recv"), rc,
                 n, ti, to, _enum(_OP, op), _enum(_ORDER, order), _stream(stream, _first(send))),
           "gc_reduce_scatter")
    return recv


def gc_all_gather(send, recv, count=None, dtype=None, stream=None):
    """All-gather: recv[d][i*count : (i+1)*count] = send[i] for every d."""
    n = len(send)
    t = _infer_dtype(send, dtype)
    cnt = _numel(send, count)
    nb = cnt * _ES.get(t, 0)
    _check(_c_ag(_bufs(send, n, nb, "send"), _bufs(recv, n, n * nb, "recv"), cnt, n, t,
                 _stream(stream, _first(send))), "gc_all_gather")
    return recv


def gc_all_to_all(send, recv, splits, row_bytes, stream=None):
    """All-to-all(v) with experts: splits is an int64 array-like [N][N][E] of rows."""
    import numpy as np
    sp = np.ascontiguousarray(np.asarray(splits, dtype=np.int64))
    if sp.ndim != 3:
        raise ValueError("splits must be [N][N][E]")
    n, _, e = sp.shape
    rb = int(row_bytes)
    rows_out = [max(0, int(x)) * rb for x in sp.clip(min=0).sum(axis=(1, 2))] if n else []
    rows_in = [max(0, int(x)) * rb for x in sp.clip(min=0).sum(axis=(0, 2))] if n else []
    _check(_c_a2a(_bufs(send, n, rows_out, "send"), _bufs(recv, n, rows_in, "recv"),
                  sp.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n, e, rb, _stream(stream, _first(send))),
           "gc_all_to_all")
    return recv


def gc_hier_all_reduce(send, recv, group_size, op="avg", order="ring", count=None, dtype=None, stream=None):
    """Two-level all-reduce over len(send) = R * group_size ranks (member i of group g = rank g*group_size + i)."""
    n = len(send)
    t = _infer_dtype(send, dtype)
    cnt = _numel(send, count)
    nb = cnt * _ES.get(t, 0)
    _check(_c_hier_ar(_bufs(send, n, nb, "send"), _bufs(recv, n, nb, "recv"), cnt, n, int(group_size), t,
                      _enum(_OP, op), _enum(_ORDER, order), _stream(stream, _first(send))), "gc_hier_all_reduce")
    return recv


def gc_hsdp_reduce_scatter(send, recv, group_size, op="avg", order="ring", recv_count=None, in_dtype=None,
                           out_dtype=None, stream=None):
    """HSDP gradient reduce-scatter: recv[r] = chunk (r mod group_size) of the reduction over all ranks."""
    n = len(send)
    rc = int(recv_count) if recv_count is not None else int(recv[0].numel())
    tin = _infer_dtype(send, in_dtype)
    tout = _infer_dtype(recv, out_dtype)
    g = max(0, int(group_size))
    _check(_c_hsdp_rs(_bufs(send, n, g * rc * _ES.get(tin, 0), "send"), _bufs(recv, n, rc * _ES.get(tout, 0), "recv"),
                      rc, n, int(group_size), tin, tout, _enum(_OP, op), _enum(_ORDER, order),
                      _stream(stream, _first(send))), "gc_hsdp_reduce_scatter")
    return recv


def _sz_array(xs):
    xs = [int(x) for x in xs]
    return (ctypes.c_size_t * max(1, len(xs)))(*xs)


def _rank_major(xs, nranks, nparams):
    """Accept [rank][param] nested lists or a flat rank-major list (returned flat), or a marshalled array."""
    if isinstance(xs, ctypes.Array):
        return xs
    if len(xs) == nranks and nparams and isinstance(xs[0], (list, tuple)):
        xs = [x for row in xs for x in row]
    if len(xs) != nranks * nparams:
        raise ValueError("need nranks * nparams pointers")
    return xs


def _shard_bytes(rows, cols, nranks, es):
    """Bytes of every (rank, parameter) dim-0 shard, rank-major (torch.chunk's rule)."""
    out = []
    for r in range(nranks):
        for nr, nc in zip(rows, cols):
            c = -(-int(nr) // nranks)
            out.append((min(int(nr), (r + 1) * c) - min(int(nr), r * c)) * int(nc) * es)
    return out


def gc_fsdp2_reduce_scatter(grads, shards, rows, cols, nranks, in_dtype, out_dtype=None, op="avg", order="ring",
                            stream=None):
    """Per-parameter Shard(0) reduce-scatter; grads / shards as [rank][param] (or flat rank-major)."""
    P, N = len(rows), int(nranks)
    out_dtype = in_dtype if out_dtype is None else out_dtype
    ti, to = _dtype_code(in_dtype), _dtype_code(out_dtype)
    g = _rank_major(grads, N, P)
    sh = _rank_major(shards, N, P)
    full = [int(nr) * int(nc) * _ES.get(ti, 0) for nr, nc in zip(rows, cols)] * max(N, 0)
    part = _shard_bytes(rows, cols, N, _ES.get(to, 0)) if N > 0 else []
    like = None if isinstance(g, ctypes.Array) else _first(g)
    _check(_c_fsdp2_rs(_bufs(g, N * P, full, "grads"), _bufs(sh, N * P, part, "shards"), _sz_array(rows),
                       _sz_array(cols), P, N, ti, to, _enum(_OP, op), _enum(_ORDER, order), _stream(stream, like)),
           "gc_fsdp2_reduce_scatter")
    return shards


def gc_fsdp2_all_gather(shards, params, rows, cols, nranks, dtype, stream=None):
    """Per-parameter Shard(0) all-gather; shards / params as [rank][param] (or flat rank-major)."""
    P, N = len(rows), int(nranks)
    t = _dtype_code(dtype)
    sh = _rank_major(shards, N, P)
    pa = _rank_major(params, N, P)
    full = [int(nr) * int(nc) * _ES.get(t, 0) for nr, nc in zip(rows, cols)] * max(N, 0)
    part = _shard_bytes(rows, cols, N, _ES.get(t, 0)) if N > 0 else []
    like = None if isinstance(pa, ctypes.Array) else _first(pa)
    _check(_c_fsdp2_ag(_bufs(sh, N * P, part, "shards"), _bufs(pa, N * P, full, "params"), _sz_array(rows),
                       _sz_array(cols), P, N, t, _stream(stream, like)), "gc_fsdp2_all_gather")
    return params


def _i64_array(xs):
    xs = [int(x) for x in xs]
    return (ctypes.c_int64 * max(1, len(xs)))(*xs)


def gc_moe_route_scratch_bytes(ntokens, topk, experts_per_rank):
    """Scratch bytes gc_moe_route needs for these per-source token counts (0 if the sizes are invalid)."""
    return int(_c_moe_scratch(_i64_array(ntokens), len(ntokens), int(topk), int(experts_per_rank)))


def _per_route(ntokens, topk, nbytes):
    return [max(0, int(t)) * max(0, int(topk)) * nbytes for t in ntokens]


def gc_moe_route(experts, ntokens, topk, experts_per_rank, splits, dest, scratch, scratch_bytes=None, stream=None):
    """MoE routing plan on the device.  experts[s]: int32 [ntokens[s] * topk] global expert ids;
    splits: int64 [N*N*E] out; dest[s]: int32 [ntokens[s] * topk * 2] (rank, row) out."""
    n = len(ntokens)
    if scratch_bytes is None:
        scratch_bytes = scratch.numel() * scratch.element_size()
    nsplit = n * n * max(0, int(experts_per_rank)) * 8
    _check(_c_moe_route(_bufs(experts, n, _per_route(ntokens, topk, 4), "experts"), _i64_array(ntokens), n,
                        int(topk), int(experts_per_rank), _buf(splits, nsplit, "splits"),
                        _bufs(dest, n, _per_route(ntokens, topk, 8), "dest"),
                        _buf(scratch, int(scratch_bytes), "scratch"), int(scratch_bytes), _stream(stream, splits)),
           "gc_moe_route")
    return splits, dest


GC_MOE_ROUTE_NOALLOC_SCRATCH_BYTES = 4 << 20


def gc_moe_route_noalloc(experts, ntokens, topk, experts_per_rank, splits, dest, stream=None):
    """gc_moe_route without a scratch argument, for callers that cannot allocate device
    memory: the plan uses the library's static per-GPU scratch (at most
    GC_MOE_ROUTE_NOALLOC_SCRATCH_BYTES; larger plans raise GcError with GC_ERR_UNSUPPORTED).
    Calls that overlap on one GPU share that scratch and race."""
    n = len(ntokens)
    nsplit = n * n * max(0, int(experts_per_rank)) * 8
    st = _c_moe_route_noalloc(_bufs(experts, n, _per_route(ntokens, topk, 4), "experts"), _i64_array(ntokens), n,
                              int(topk), int(experts_per_rank), _buf(splits, nsplit, "splits"),
                              _bufs(dest, n, _per_route(ntokens, topk, 8), "dest"), _stream(stream, splits))
    if st == GC_ERR_UNSUPPORTED:
        need = gc_moe_route_scratch_bytes(ntokens, topk, experts_per_rank)
        if need > GC_MOE_ROUTE_NOALLOC_SCRATCH_BYTES:
            raise GcError(st, f"gc_moe_route_noalloc (the plan needs {need} bytes of scratch, the static scratch "
                              f"holds {GC_MOE_ROUTE_NOALLOC_SCRATCH_BYTES}; use gc_moe_route with a scratch buffer)")
    _check(st, "gc_moe_route_noalloc")
    return splits, dest


def gc_moe_dispatch(tokens, ntokens, dest, topk, row_bytes, recv, recv_rows, stream=None):
    """Copy every token row of every source to the receive rows its routes name."""
    n, rb = len(ntokens), int(row_bytes)
    _check(_c_moe_dispatch(_bufs(tokens, n, [max(0, int(t)) * rb for t in ntokens], "tokens"), _i64_array(ntokens),
                           _bufs(dest, n, _per_route(ntokens, topk, 8), "dest"), n, int(topk), rb,
                           _bufs(recv, n, [max(0, int(r)) * rb for r in recv_rows], "recv"), _i64_array(recv_rows),
                           _stream(stream, _first(recv))), "gc_moe_dispatch")
    return recv


def gc_moe_combine(expert_out, expert_rows, dest, weights, ntokens, topk, hidden, dtype, out, stream=None):
    """out[s][t] = sum_k weights[s][t*topk + k] * expert_out[rank][row] over the routes of token t."""
    n, t = len(ntokens), _dtype_code(dtype)
    rb = max(0, int(hidden)) * _ES.get(t, 0)
    _check(_c_moe_combine(_bufs(expert_out, n, [max(0, int(r)) * rb for r in expert_rows], "expert_out"),
                          _i64_array(expert_rows), _bufs(dest, n, _per_route(ntokens, topk, 8), "dest"),
                          _bufs(weights, n, _per_route(ntokens, topk, 4), "weights"), _i64_array(ntokens), n,
                          int(topk), int(hidden), t, _bufs(out, n, [max(0, int(x)) * rb for x in ntokens], "out"),
                          _stream(stream, _first(out))), "gc_moe_combine")
    return out


# ------------------------------------------------------------------ HBM layout

def gc_rank_buffers(nranks, count, dtype, device="cuda", stagger_bytes=4096, slot_align=2 << 20):
    """N rank buffers of `count` elements carved from one device allocation.

    Rank r starts at r * (slot + stagger_bytes) bytes, slot = the buffer size
    rounded up to slot_align.  Every element offset then sits at a different
    position modulo slot_align on each rank, so the N same-offset accesses a
    reduction makes at once fall into different HBM channels and banks instead
    of piling onto one.  On MI355X a 4 KiB stagger raised the 8 x 64 MiB bf16
    all-reduce from about 5.6 to 5.8 TB/s.  Returns a list of 1-D views.
    """
    import torch
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32, "int32": torch.int32}.get(dtype, dtype)
    es = torch.empty((), dtype=tdt).element_size()
    slot = -(-count * es // slot_align) * slot_align
    step = slot + stagger_bytes
    if step % es:
        raise ValueError("stagger_bytes must be a multiple of the element size")
    total = (nranks - 1) * step + count * es
    slab = torch.empty(max(1, total // es), dtype=tdt, device=device)
    return [slab[r * step // es: r * step // es + count] for r in range(nranks)]


class RankArena:
    """Per-rank HBM regions for N ranks on one GPU: every rank owns one region,
    as a real rank owns its GPU's memory, and all of a rank's buffers are
    bump-allocated inside it at the same offset on every rank.

    The regions are carved from one allocation; rank r's region starts at
    r * (region_bytes + stagger_bytes).  A collective reads and writes the same
    offset on all N ranks at once; regions a large power of two apart plus a
    small stagger spread those N streams over HBM's channels and stacks.  On
    MI355X, 16 GiB regions raised the 8 x 64 MiB bf16 all-reduce from about 5.8
    to 6.2 TB/s and 32 GiB regions by up to 1.7 % more (every 8-rank workload
    gained 0.4-1.1 %); 4 GiB regions raised the 64-rank all-gather from about
    5.4 to 6.7 TB/s.

    region_bytes=None picks the largest power of two up to max_region for which
    all N regions fit in free device memory (keeping reserve_bytes free), and at
    least min_bytes.
    """

    def __init__(self, nranks, region_bytes=None, stagger_bytes=4096, min_bytes=0, device="cuda",
                 reserve_bytes=4 << 30, max_region=32 << 30):
        import torch
        self.nranks = int(nranks)
        self.stagger = int(stagger_bytes)
        if region_bytes is None:
            free = torch.cuda.mem_get_info(torch.device(device))[0] if str(device).startswith("cuda") else 1 << 40
            region_bytes = 1 << 21
            while (region_bytes * 2 <= max_region and
                   self.nranks * (region_bytes * 2 + self.stagger) <= free - reserve_bytes):
                region_bytes *= 2
            while region_bytes < min_bytes:
                region_bytes *= 2
        self.region = int(region_bytes)
        self.step = self.region + self.stagger
        self.slab = torch.empty(self.nranks * self.step, dtype=torch.uint8, device=device)
        self.used = 0

    def alloc(self, count, dtype):
        """One buffer of `count` elements per rank, at the same offset of every region."""
        import torch
        tdt = {"bf16": torch.bfloat16, "fp32": torch.float32, "int32": torch.int32}.get(dtype, dtype)
        es = torch.empty((), dtype=tdt).element_size()
        nbytes = int(count) * es
        if self.used + nbytes > self.region:
            raise MemoryError(f"rank region of {self.region} bytes is full")
        out = [self.slab[r * self.step + self.used: r * self.step + self.used + nbytes].view(tdt)
               for r in range(self.nranks)]
        self.used += -(-nbytes // 256) * 256
        return out


# ------------------------------------------------------------------ bucket plan

def gc_bucket_plan_create(numels, dtype, cap_bytes, reverse=True, pad_to=1):
    arr = (ctypes.c_size_t * max(1, len(numels)))(*[int(x) for x in numels])
    out = ctypes.c_void_p()
    _check(_c_plan_create(arr, len(numels), _dtype_code(dtype), int(cap_bytes), int(bool(reverse)), int(pad_to),
                          ctypes.byref(out)), "gc_bucket_plan_create")
    return out.value


def gc_bucket_plan_query(plan, ntensors):
    nb = ctypes.c_int()
    _check(_c_plan_query(plan, ctypes.byref(nb), None, None, None), "gc_bucket_plan_query")
    bucket_numel = (ctypes.c_size_t * max(1, nb.value))()
    tb = (ctypes.c_int * max(1, ntensors))()
    to = (ctypes.c_size_t * max(1, ntensors))()
    _check(_c_plan_query(plan, ctypes.byref(nb), bucket_numel, tb, to), "gc_bucket_plan_query")
    return (nb.value, [bucket_numel[i] for i in range(nb.value)], [tb[i] for i in range(ntensors)],
            [to[i] for i in range(ntensors)])


def gc_bucket_plan_destroy(plan):
    _c_plan_destroy(plan)


def gc_bucket_pack(plan, bucket, tensors, bucket_bufs, nranks, stream=None):
    """tensors: flat rank-major list of nranks*ntensors tensors (or None for tensors outside the bucket).
    The plan handle does not carry the tensor sizes, so only device and layout are checked here
    (BucketPlan.pack checks sizes too)."""
    _check(_c_pack(plan, int(bucket), _bufs(tensors, 0, 0, "tensors"), _bufs(bucket_bufs, 0, 0, "bucket_bufs"),
                   int(nranks), _stream(stream, _first(bucket_bufs))), "gc_bucket_pack")


def gc_bucket_unpack(plan, bucket, bucket_bufs, tensors, nranks, stream=None):
    _check(_c_unpack(plan, int(bucket), _bufs(bucket_bufs, 0, 0, "bucket_bufs"), _bufs(tensors, 0, 0, "tensors"),
                     int(nranks), _stream(stream, _first(bucket_bufs))), "gc_bucket_unpack")


def gc_bucket_all_reduce(plan, bucket, tensors, nranks, op="avg", order="ring", sumsq=None, stream=None):
    """Zero-copy all-reduce of one bucket, in place over the tensors (rank-major flat list).
    sumsq: optional CUDA float64 tensor (one element) that receives += sum of squared results."""
    _check(_c_bucket_ar(plan, int(bucket), _bufs(tensors, 0, 0, "tensors"), int(nranks), _enum(_OP, op),
                        _enum(_ORDER, order), _buf(sumsq, 8, "sumsq"), _stream(stream, _first(tensors))),
           "gc_bucket_all_reduce")


class BucketPlan:
    """Owns a gc_bucket_plan handle and caches its query results.  Its calls
    check every tensor and bucket buffer against the plan's sizes before the
    library sees the pointers."""

    def __init__(self, numels, dtype, cap_bytes, reverse=True, pad_to=1):
        self.numels = [int(x) for x in numels]
        self.reverse = bool(reverse)
        self.es = _ES.get(_dtype_code(dtype), 0)
        self.handle = gc_bucket_plan_create(self.numels, dtype, cap_bytes, reverse, pad_to)
        self.nbuckets, self.bucket_numel, self.tensor_bucket, self.tensor_offset = gc_bucket_plan_query(
            self.handle, len(self.numels))

    def bucket_tensors(self, b):
        """Tensor indices of bucket b in packing order (an empty tensor shares its
        offset with the next one, so ties follow the visiting order)."""
        ts = [t for t in range(len(self.numels)) if self.tensor_bucket[t] == b]
        return sorted(ts, key=lambda t: (self.tensor_offset[t], -t if self.reverse else t))

    def _tensors(self, bucket, tensors, nranks):
        """Checked pointer array of the rank-major tensor list: bucket members need their full size."""
        if isinstance(tensors, ctypes.Array):        # marshalled once by gc_pointers: only its length is checked
            return _bufs(tensors, max(0, nranks) * len(self.numels), 0, "tensors")
        need = [n * self.es if self.tensor_bucket[t] == bucket else 0 for t, n in enumerate(self.numels)]
        return _bufs(tensors, max(0, nranks) * len(need), need * max(0, nranks), "tensors")

    def _bucket_bufs(self, bucket, bufs, nranks):
        nb = self.bucket_numel[bucket] * self.es if 0 <= bucket < self.nbuckets else 0
        return _bufs(bufs, max(0, nranks), nb, "bucket_bufs")

    def pack(self, bucket, tensors, bucket_bufs, nranks, stream=None):
        stream = _stream(stream, _first(bucket_bufs))
        gc_bucket_pack(self.handle, bucket, self._tensors(bucket, tensors, nranks),
                       self._bucket_bufs(bucket, bucket_bufs, nranks), nranks, stream)

    def unpack(self, bucket, bucket_bufs, tensors, nranks, stream=None):
        stream = _stream(stream, _first(bucket_bufs))
        gc_bucket_unpack(self.handle, bucket, self._bucket_bufs(bucket, bucket_bufs, nranks),
                         self._tensors(bucket, tensors, nranks), nranks, stream)

    def all_reduce(self, bucket, tensors, nranks, op="avg", order="ring", sumsq=None, stream=None):
        stream = _stream(stream, _first(tensors))
        gc_bucket_all_reduce(self.handle, bucket, self._tensors(bucket, tensors, nranks), nranks, op, order, sumsq,
                             stream)

    def close(self):
        if self.handle:
            gc_bucket_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
