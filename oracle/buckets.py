"""DDP gradient buckets and FSDP FlatParameter layout (test infrastructure only).

Bucket assignment (AIG6 §6.2.4 "Reducer 与梯度桶化"; NXMR §5.1): gradients
are grouped into buckets of a fixed capacity (25 MB by default), filled in the
order backward produces gradients, i.e. the reverse of the model's definition
order, and a bucket is all-reduced as soon as it is full.  Readings where the
pages are silent:
  * "full" means the bucket's bytes reached the capacity: a tensor is appended
    to the open bucket, and the bucket closes once its bytes are >= capacity;
  * a tensor is never split across buckets;
  * the last, partly filled bucket is closed at the end;
  * no special small first bucket and no alignment padding.

Bucket layout (DTLM §4 FSDP1 "1D FlatParameter 是怎么创建的"): the tensors are
concatenated in bucket order; tensor t occupies [offset_t, offset_t + numel_t)
with offsets the running sums of numels.  For a FlatParameter the total is
padded with zeros up to a multiple of the world size, and rank i's shard is the
i-th of N equal slices.
"""

import numpy as np


def assign_buckets(numels, elem_bytes, cap_bytes, reverse=True):
    """List of buckets, each a list of tensor indices in packing order."""
    order = range(len(numels) - 1, -1, -1) if reverse else range(len(numels))
    buckets, current, current_bytes = [], [], 0
    for t in order:
        current.append(t)
        current_bytes += int(numels[t]) * elem_bytes
        if current_bytes >= cap_bytes:
            buckets.append(current)
            current, current_bytes = [], 0
    if current:
        buckets.append(current)
    return buckets


def bucket_layout(bucket, numels, pad_to=1):
    """(offsets, used, padded): per-tensor offsets, elements used, total after padding."""
    offsets, run = [], 0
    for t in bucket:
        offsets.append(run)
        run += int(numels[t])
    padded = -(-run // pad_to) * pad_to if pad_to > 1 else run
    return offsets, run, padded


def pack(tensors, bucket, numels, pad_to=1):
    """Concatenate one rank's tensors of a bucket into a flat buffer (zero padding at the end)."""
    offsets, used, padded = bucket_layout(bucket, numels, pad_to)
    dt = np.asarray(tensors[bucket[0]]).dtype if bucket else np.uint16
    flat = np.zeros(padded, dtype=dt)
    for t, off in zip(bucket, offsets):
        src = np.asarray(tensors[t]).reshape(-1)
        if src.size != int(numels[t]):
            raise ValueError("tensor size does not match the plan")
        flat[off:off + src.size] = src
    return flat


def unpack(flat, bucket, numels):
    """Inverse of pack: dictionary tensor index -> 1-D copy of its slice of the flat buffer."""
    offsets, _, _ = bucket_layout(bucket, numels)
    return {t: np.asarray(flat)[off:off + int(numels[t])].copy() for t, off in zip(bucket, offsets)}


def flat_param_shards(numels, world_size):
    """FlatParameter: tensor intervals in the flat buffer, padded size, and each rank's shard range."""
    bucket = list(range(len(numels)))
    offsets, used, padded = bucket_layout(bucket, numels, world_size)
    intervals = [(o, o + int(n)) for o, n in zip(offsets, numels)]
    per = padded // world_size
    shards = [(i * per, (i + 1) * per) for i in range(world_size)]
    return intervals, used, padded, shards


def uneven_dim0_shards(rows, world_size):
    """Dim-0 shards of a parameter when world_size does not divide its rows.

    Follows the torch.chunk-like rule of DTLM §4 (FSDP2, uneven Shard(0)):
    every rank gets ceil(rows / world_size) rows except trailing ranks, which
    get fewer or none.
    """
    c = -(-rows // world_size) if rows else 0
    return [(min(rows, i * c), min(rows, (i + 1) * c)) for i in range(world_size)]


def bucket_all_reduce(per_rank_tensors, bucket, numels, dtype, op="avg", order="ring", pad_to=1):
    """Zero-copy bucketed all-reduce, defined as its plain composition: pack the
    bucket on every rank, all-reduce the packed buffers (padding included), and
    unpack.  Returns per rank a dict tensor index -> reduced values.
    (AIG6 §6.2.4: gradient_as_bucket_view makes the bucket the gradients'
    storage; the reduction itself is the bucket's all-reduce.)"""
    from .collectives import all_reduce
    flats = [pack(per_rank_tensors[r], bucket, numels, pad_to) for r in range(len(per_rank_tensors))]
    reduced = all_reduce(flats, dtype, op, order)
    return [unpack(reduced[r], bucket, numels) for r in range(len(reduced))]


def sum_of_squares(values, dtype):
    """Exact sum of squared element values (a Fraction), for gradient-norm
    clipping after the sync (AIG6 §6.8.1: clip_grad_norm_ on the synced gradients).
    bf16 values are given as bit patterns."""
    from fractions import Fraction
    from .numerics import bf16_to_f32
    v = bf16_to_f32(values) if dtype == "bf16" else np.asarray(values, dtype=np.float32)
    total = Fraction(0)
    for x in v.astype(np.float64):
        f = Fraction(float(x))
        total += f * f
    return total
