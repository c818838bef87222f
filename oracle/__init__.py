"""Reference oracle for the gradient-synchronisation collectives.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this package: only the test-suite, the smoke check and the CPU-baseline leg of
the benchmark use it.  It shares no code with the HIP library (no kernels,
headers, helpers, tables or constants) and never reads a value the GPU produced.

It is a plain, slow, single-threaded CPU implementation written from the pages
that define the method.  Pages are cited by these short names:

  DTLM   "Distributed Training for Large Models: Collectives, FSDP/ZeRO,
         DeviceMesh, and Multi-Dimensional Parallelism" (zexinliu.github.io).
  AIG6   "AI Infra Guide", chapter 6 "分布式训练基础" (theaiera.top).
  NXMR   the nxmr.cn article on collective communication and model
         parallelism (news/160867); cited by its own section numbers.

Floating point: the pages fix the reduction precision at fp32
(AIG6 §6.3.4, MixedPrecision(reduce_dtype=torch.float32)), so partial sums are
numpy float32 values and every add is one IEEE-754 fp32 add.  Integer data
wraps modulo 2**32.

Modules
  numerics     bf16 <-> fp32 (round to nearest, ties to even)
  collectives  owner chunks, ring reduce-scatter / all-gather / all-reduce
               emulated step by step with traffic counters, rank-order fold,
               exact brute-force sum, all-to-all(v)
  buckets      DDP bucket assignment, bucket pack / unpack, FlatParameter
               flatten / pad / shard, zero-copy bucket all-reduce, sum of squares
  fsdp2        FSDP2 per-parameter Shard(0) reduce-scatter / all-gather with
               uneven and empty shards
  hierarchical two-level all-reduce over rank groups and the HSDP gradient
               reduce-scatter
  moe          expert-parallel MoE around the all-to-all: routing plan,
               dispatch from token order, weighted combine back to token order
  sampled      evaluation of single output elements, for checks at sizes the
               step-by-step emulation cannot hold in memory
  cost_model   the pages' alpha-beta estimates (context numbers)

Parity status: every function here is pinned by a CPU test (tests/test_oracle_*)
against the pages' worked examples, closed forms, library routines or brute
force, except the points the pages leave open (bucket closing rule, MoE routing
details, the order and rounding of the MoE combine); those are readings,
recorded as such, pinned by hand-worked examples and the invariants they must
satisfy.
"""

from . import numerics, collectives, buckets, sampled, cost_model, moe, fsdp2, hierarchical  # noqa: F401
