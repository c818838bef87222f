"""Pins for the oracle's bf16 conversions against the IEEE definition and a library routine."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.numerics import bf16_to_f32, bf16_ulp_distance, f32_to_bf16


def _bf16_value(bits):
    """Exact rational value of a finite bf16 bit pattern, from the IEEE layout (sign, 8-bit exp, 7-bit frac)."""
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0:
        return sign * Fraction(frac, 1 << 7) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(frac, 1 << 7)) * (Fraction(2) ** (exp - 127))


def _nearest_even_bruteforce(x):
    """bf16 bits nearest to finite fp32 x by exhaustive comparison with its two bf16 neighbours."""
    v = Fraction(float(x))
    bits = int(np.float32(x).view(np.uint32))
    lo = bits >> 16                                   # truncation toward zero (same sign)
    cands = [lo, lo + 1] if (bits & 0xFFFF) else [lo]
    best = None
    for c in cands:
        if (c & 0x7FFF) >= 0x7F80:                   # rounds past the largest finite bf16
            # overflow: the carry reaches the infinity pattern; judge against 2^128
            cv = Fraction(2) ** 128 * (-1 if c & 0x8000 else 1)
        else:
            cv = _bf16_value(c)
        d = abs(cv - v)
        key = (d, c & 1)                              # ties resolved toward an even last bit
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def _special_inputs():
    f = [0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875,          # exact ties (dropped bits == 0x8000)
         3.4028234663852886e38, -3.4028234663852886e38,         # fp32 max -> overflows to inf in bf16
         3.3895313892515355e38,                                  # largest finite bf16
         1e-45, -1e-45, 1.1754942e-38, 1.1754944e-38,            # subnormals / smallest normal
         np.inf, -np.inf]
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x00018000, 0x7F7F8000, 0x7F7E8000],
                    dtype=np.uint32).view(np.float32)
    return np.concatenate([np.array(f, dtype=np.float32), ties])


def test_f32_to_bf16_matches_definition_exhaustively_on_samples():
    rng = np.random.default_rng(0)
    rand_bits = rng.integers(0, 2**32, size=4000, dtype=np.uint64).astype(np.uint32)
    vals = np.concatenate([_special_inputs(), rand_bits.view(np.float32)])
    vals = vals[np.isfinite(vals)]
    got = f32_to_bf16(vals)
    for x, g in zip(vals, got):
        assert int(g) == _nearest_even_bruteforce(x), (x, hex(int(g)))


def test_f32_to_bf16_matches_torch_rne():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    vals = np.concatenate([_special_inputs(), bits.view(np.float32)])
    ours = f32_to_bf16(vals)
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(vals)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays NaN, keeps its sign, is quiet
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all(ours[nan] & 0x0040)
    assert np.array_equal(ours[nan] >> 15, (vals[nan].view(np.uint32) >> 31).astype(np.uint16))


def test_bf16_to_f32_is_exact_widening():
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = bf16_to_f32(allbits)
    ref = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    # round trip of every non-NaN pattern is the identity
    nn = ~np.isnan(ours)
    assert np.array_equal(f32_to_bf16(ours[nn]), allbits[nn])


def test_ulp_distance():
    one = f32_to_bf16(np.float32(1.0)).reshape(1)
    nxt = (one + 1).astype(np.uint16)
    assert bf16_ulp_distance(one, nxt)[0] == 1
    assert bf16_ulp_distance(np.array([0x0000], np.uint16), np.array([0x8000], np.uint16))[0] == 0
    # across zero: smallest positive and smallest negative subnormal are 2 apart
    assert bf16_ulp_distance(np.array([0x0001], np.uint16), np.array([0x8001], np.uint16))[0] == 2
    assert bf16_ulp_distance(np.array([0x7FC0], np.uint16), np.array([0xFFC1], np.uint16))[0] == 0
    assert bf16_ulp_distance(np.array([0x7FC0], np.uint16), np.array([0x3F80], np.uint16))[0] > 1000


@pytest.mark.parametrize("x,expect", [(1.0, 0x3F80), (-2.0, 0xC000), (np.inf, 0x7F80)])
def test_f32_to_bf16_known_patterns(x, expect):
    assert int(f32_to_bf16(np.float32(x)).reshape(-1)[0]) == expect
