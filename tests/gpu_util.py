"""Helpers for GPU tests: numpy <-> torch CUDA transfers with bf16 carried as uint16 bit patterns."""

import numpy as np
import torch

from oracle.numerics import bf16_ulp_distance

DEV = torch.device("cuda:0")
TORCH = {"bf16": torch.bfloat16, "fp32": torch.float32, "int32": torch.int32}


def to_dev(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)
    if dtype == "fp32":
        return torch.from_numpy(a.astype(np.float32)).to(DEV)
    return torch.from_numpy(a.astype(np.int32)).to(DEV)


def from_dev(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def empty(n, dtype):
    return torch.empty(n, dtype=TORCH[dtype], device=DEV)


def assert_same(got, want, dtype, what=""):
    """Bit-exact comparison; NaN matches NaN of any payload (bf16 and fp32)."""
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if dtype == "bf16":
        from oracle.numerics import bf16_is_nan
        both_nan = bf16_is_nan(got) & bf16_is_nan(want)
        bad = np.nonzero((got != want) & ~both_nan)[0]
    elif dtype == "fp32":
        gb, wb = got.view(np.uint32), want.view(np.uint32)
        both_nan = np.isnan(got) & np.isnan(want)
        bad = np.nonzero((gb != wb) & ~both_nan)[0]
    else:
        bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: got {got[bad[:5]]} want {want[bad[:5]]}"


def max_ulp(got, want):
    d = bf16_ulp_distance(got, want)
    return int(d.max()) if d.size else 0
