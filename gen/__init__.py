"""Seeded synthetic inputs shared by the tests, the oracle checks and the benchmark.

This package holds input generation only: none of the collectives' arithmetic
(no folds, no averaging, no bf16 round-to-nearest, no chunking, no bucket or
all-to-all layout of the method).  It is the one piece the CPU oracle and the
HIP library both consume.

Counter-based generator.  Every value is a pure function of
(seed, rank, stream, index), so any element of a multi-gigabyte rank buffer can
be recomputed on the host from its index alone, and the device twin
(gen/device.hip) produces the identical bits in HBM.

  mix64(z)     SplitMix64's output function (Steele, Lea & Flood, "Fast
               splittable pseudorandom number generators", OOPSLA 2014):
                 z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
                 z = (z ^ (z >> 27)) * 0x94D049BB133111EB
                 z ^ (z >> 31)                         (all mod 2**64)
  key          mix64(seed + rank) ^ mix64(stream + 0x9E3779B97F4A7C15)
               (the offset keeps (rank, stream) and (stream, rank) apart)
  U64(i, m)    mix64(key + (4*i + m) * 0x9E3779B97F4A7C15), m in 0..3

Distributions (each exact in integer or correctly-rounded double arithmetic,
so host and device agree bit for bit):
  uniform_f32  ((U64(i,0) >> 40) - 2**23) * 2**-23       in [-1, 1), exact
  normal       Irwin-Hall(4): z = (sum_m (U64(i,m) >> 32) * 2**-32 - 2) * sqrt(3)
               (unit variance, bell-shaped, bounded at +-3.46 sigma); the sum and
               the shift are exact in double, the one rounding is the product
               with the host-computed double sqrt(3)*sigma, then double -> fp32
               (round to nearest even, done by the conversion instruction).
  normal bf16  the fp32 value's top 16 bits (truncation toward zero).  This is a
               property of the synthetic distribution only; it deliberately is
               not the collectives' round-to-nearest rule.
  int32        the top 32 bits of U64(i, 0), as a two's-complement int32.
"""

from .host import (  # noqa: F401
    GOLDEN, MASK64, mix64, stream_key, u64, uniform_f32, normal_f32, normal_bf16, int32_values,
)
