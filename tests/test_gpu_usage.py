"""The usage example of the package, run as written and checked: N ranks as N
buffers in one GPU's HBM; all-reduce, FSDP reduce-scatter / all-gather, a
zero-copy DDP bucket all-reduce, and the MoE route -> dispatch -> combine
chain.  Each result is checked against the oracle or an identity that holds
for it."""

import numpy as np
import pytest
import torch

import collective_communication_reduction_amd as gc
from oracle import buckets as OB
from oracle import collectives as C
from tests.gpu_util import assert_same, from_dev

pytestmark = pytest.mark.gpu


def test_usage_example():
    # --- the example ------------------------------------------------------
    N, S = 8, 1 << 20
    arena = gc.RankArena(N, region_bytes=1 << 30)           # one HBM region per rank
    grads = arena.alloc(S, "bf16")                           # N views, one per rank
    for r, g in enumerate(grads):
        g.copy_(torch.randn(S, generator=torch.Generator().manual_seed(r)).mul_(1e-3).bfloat16())
    avg = arena.alloc(S, "bf16")
    gc.gc_all_reduce(grads, avg, op="avg")                   # ring order, fp32 partials, one rounding

    shards = arena.alloc(S // N, "fp32")                     # FSDP: bf16 gradients -> fp32 shards
    gc.gc_reduce_scatter(grads, shards, op="avg")
    params = arena.alloc(S // N, "bf16")
    for p, s in zip(params, shards):
        p.copy_(s.bfloat16())                                # (an optimizer step would go here)
    gathered = arena.alloc(S, "bf16")
    gc.gc_all_gather(params, gathered)

    numels = [300_000, 4096, 700_000, 44_480]                # DDP: tensors of one rank, model order
    plan = gc.BucketPlan(numels, "bf16", cap_bytes=1 << 20)  # buckets filled in reverse order
    tensors = [t for r in range(N) for t in torch.split(grads[r], numels)]
    ptrs = gc.gc_pointers(tensors)                           # marshal once, reuse every step
    for b in range(plan.nbuckets):
        plan.all_reduce(b, ptrs, N, op="avg")                # in place over the tensors
    buckets = [plan.bucket_tensors(b) for b in range(plan.nbuckets)]
    plan.close()

    E, K, T, H = 2, 2, 1000, 512                             # MoE: 2 experts per rank, top-2
    rng = torch.Generator(device="cuda").manual_seed(7)
    experts = [torch.randint(0, N * E, (T, K), dtype=torch.int32, device="cuda", generator=rng) for _ in range(N)]
    for e in experts:
        e[:, 1] = (e[:, 0] + 1) % (N * E)                    # two distinct experts per token
    tokens = [torch.randn(T, H, device="cuda", generator=rng).bfloat16() for _ in range(N)]
    splits = torch.empty(N * N * E, dtype=torch.int64, device="cuda")
    dest = [torch.empty(T * K * 2, dtype=torch.int32, device="cuda") for _ in range(N)]
    scratch = torch.empty(gc.gc_moe_route_scratch_bytes([T] * N, K, E), dtype=torch.uint8, device="cuda")
    gc.gc_moe_route(experts, [T] * N, K, E, splits, dest, scratch)
    rows = splits.view(N, N, E).sum(dim=(0, 2)).tolist()     # receive rows per rank
    recv = [torch.empty(max(1, n) * H, dtype=torch.bfloat16, device="cuda") for n in rows]
    gc.gc_moe_dispatch(tokens, [T] * N, dest, K, H * 2, recv, rows)
    weights = [torch.full((T * K,), 0.5, device="cuda") for _ in range(N)]   # identity experts
    out = [torch.empty(T, H, dtype=torch.bfloat16, device="cuda") for _ in range(N)]
    gc.gc_moe_combine(recv, rows, dest, weights, [T] * N, K, H, "bf16", out)
    torch.cuda.synchronize()
    # --- checks -------------------------------------------------------------
    host = [from_dev(x) for x in gc_inputs(N, S)]            # the example's gradients, regenerated
    want_avg = C.all_reduce(host, "bf16", "avg", "ring")[0]
    for r in (0, N - 1):
        assert_same(from_dev(avg[r]), want_avg, "bf16", f"all-reduce rank {r}")
    want_shards = C.reduce_scatter(host, "bf16", "fp32", "avg", "ring")
    for j in (0, N - 1):
        assert_same(from_dev(shards[j]), want_shards[j], "fp32", f"shard {j}")
    whole = torch.cat(params)
    for r in (0, N - 1):
        assert torch.equal(gathered[r].view(torch.int16), whole.view(torch.int16)), f"all-gather rank {r}"
    offs = np.concatenate([[0], np.cumsum(numels)])
    per_rank = [[h[offs[t]:offs[t + 1]] for t in range(len(numels))] for h in host]
    for bucket in buckets:                                   # in-place bucket sync, each bucket its own ring
        want = OB.bucket_all_reduce(per_rank, bucket, numels, "bf16", "avg", "ring")
        for t in bucket:
            for r in (0, N - 1):
                assert_same(from_dev(tensors[r * len(numels) + t]), want[r][t], "bf16", f"bucket tensor {t}")
    for s in range(N):                                       # 0.5 x + 0.5 x == x exactly
        assert torch.equal(out[s].view(torch.int16), tokens[s].view(torch.int16)), f"MoE source {s}"


def gc_inputs(N, S):
    """The example's gradients, regenerated on the host."""
    return [torch.randn(S, generator=torch.Generator().manual_seed(r)).mul_(1e-3).bfloat16() for r in range(N)]
