"""Host (numpy) side of the counter-based input generator; see the package docstring."""

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def mix64(z):
    """SplitMix64 output function on uint64 arrays (wraps mod 2**64)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed, rank, stream):
    seed, rank, stream = int(seed), int(rank), int(stream)
    a = int(mix64(np.uint64((seed + rank) & MASK64)))
    b = int(mix64(np.uint64((stream + GOLDEN) & MASK64)))
    return (a ^ b) & MASK64


def u64(key, idx, m):
    """U64(i, m) for an array of indices i."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        ctr = np.uint64(key) + (idx * np.uint64(4) + np.uint64(m)) * np.uint64(GOLDEN)
    return mix64(ctr)


def uniform_f32(key, idx):
    top = (u64(key, idx, 0) >> np.uint64(40)).astype(np.int64)
    return ((top - (1 << 23)).astype(np.float64) * 2.0 ** -23).astype(np.float32)


def normal_f32(key, idx, sigma):
    s = np.zeros(np.shape(idx), dtype=np.uint64)
    for m in range(4):
        s = s + (u64(key, idx, m) >> np.uint64(32))
    z = s.astype(np.float64) * 2.0 ** -32 - 2.0
    scale = np.float64(np.sqrt(3.0)) * np.float64(sigma)
    return (z * scale).astype(np.float32)


def normal_bf16(key, idx, sigma):
    """bf16 bit patterns: top half of the fp32 normal value (see package docstring)."""
    f = np.ascontiguousarray(normal_f32(key, idx, sigma))
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def normal_scale(sigma):
    """The double sqrt(3)*sigma both generator sides multiply by."""
    return float(np.float64(np.sqrt(3.0)) * np.float64(sigma))


def int32_values(key, idx):
    return (u64(key, idx, 0) >> np.uint64(32)).astype(np.uint32).view(np.int32)
