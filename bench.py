"""Benchmark of the gradient-sync collectives on one MI355X.

Default: the all-reduce the headline metric is quoted on, 8 ranks x 33,554,432
bf16 elements (64 MiB each), averaged in fp32, rounded to bf16, ring fold
order, fused single-pass kernel.  One step = one all-reduce of one batch of
rank buffers.  Inputs are generated on the device (seeded, synthetic) before
the timed region and rotated over several replicas so that consecutive steps
never find their data in the 256 MB MALL.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

Prints one JSON line.  value = algorithmic bytes per step / time per step
(every input read once, every output written once), in GB/s; roofline.frac
is the dominant kernel's achieved bandwidth over the 8 TB/s HBM3E peak.

Other workloads (--workload): ar_fp32_n4, ddp_llama7b, ddp_llama7b_zero_copy,
fsdp_layer_n64, moe_a2a_n8 (the remaining parity configurations, measured the
same way; the zero-copy DDP step all-reduces each bucket in place over the
gradient tensors instead of packing and unpacking it), and moe_ep_n8 (the
expert-parallel MoE data flow: routing plan, dispatch from token order and
weighted combine back to token order, identity experts), and fsdp2_layer_n64
(the FSDP layer sharded per parameter on dim 0, as FSDP2 does), hier_ar_n16
(the two-level all-reduce of 16 ranks as two groups of eight), and hsdp_layer_n16
(the HSDP step of the same layer on that mesh: reduce-scatter over all 16 ranks,
all-gather inside each group).  --algo rs_ag and --order rank / ring_wire time the
all-reduce workloads' other algorithm and fold orders.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "effective HBM GB/s (% of peak) for N=8 × 64 MiB bf16 all-reduce on 1 MI355X"
CSRC = "collective_communication_reduction_amd/csrc/"
# Sources of each workload's dominant kernel: a committed profile's counters
# stay valid while these files hash to the value recorded with them.
KERNEL_SOURCES = {
    "reduce": [CSRC + "reduce.hip", CSRC + "fold.h", CSRC + "device_common.h"],
    "bucket": [CSRC + "bucket.hip", CSRC + "fold.h", CSRC + "device_common.h"],
    "a2a": [CSRC + "movement.hip", CSRC + "device_common.h"],
    "moe": [CSRC + "moe.hip", CSRC + "fold.h", CSRC + "device_common.h"],
    "hier": [CSRC + "hier.hip", CSRC + "fold.h", CSRC + "device_common.h"],
}
WORKLOAD_KERNELS = {"ar_bf16_n8": "reduce", "ar_fp32_n4": "reduce", "ddp_llama7b": "reduce",
                    "fsdp_layer_n64": "reduce", "ddp_llama7b_zero_copy": "bucket", "moe_a2a_n8": "a2a",
                    "moe_ep_n8": "moe", "fsdp2_layer_n64": "reduce", "hier_ar_n16": "hier",
                    "hsdp_layer_n16": "hier"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="ar_bf16_n8",
                   choices=["ar_bf16_n8", "ar_fp32_n4", "ddp_llama7b", "ddp_llama7b_zero_copy", "fsdp_layer_n64",
                            "moe_a2a_n8", "moe_ep_n8", "fsdp2_layer_n64", "hier_ar_n16", "hsdp_layer_n16"])
    p.add_argument("--algo", default="fused", choices=["fused", "rs_ag"],
                   help="all-reduce workloads: fused single pass, or reduce-scatter to a scratch shard then all-gather")
    p.add_argument("--order", default="ring", choices=["ring", "rank", "ring_wire"],
                   help="all-reduce workloads: fold order (ring; rank 0..N-1; ring with bf16 partials on the wire)")
    p.add_argument("--replicas", type=int, default=4)
    p.add_argument("--layout", default="arena", choices=["arena", "staggered", "separate"],
                   help="placement of the rank buffers in HBM")
    p.add_argument("--stagger", type=int, default=None,
                   help="extra bytes between consecutive ranks' memory (default: the workload's, else 4096)")
    p.add_argument("--max-region", type=int, default=32, metavar="GIB",
                   help="largest per-rank region of the rank arena (a power of two, GiB)")
    p.add_argument("--region-bytes", type=int, default=None, metavar="BYTES",
                   help="exact per-rank region of the rank arena (ranks are region + stagger bytes apart)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-copy-ceiling", action="store_true", help="skip the 2 GiB copy-ceiling measurement")
    p.add_argument("--no-extras", action="store_true",
                   help="the default workload only: skip the other configurations' extra keys")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="also launch a plain device copy of this many MiB (counter calibration runs)")
    p.add_argument("--patterns", action="store_true",
                   help="instead of the bench line: each dominant kernel beside the unordered access pattern of "
                        "its own reads and writes (bench_patterns.hip) on the same buffers")
    return p.parse_args()


def kernel_hash(workload):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[WORKLOAD_KERNELS[workload]]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload):
    """HBM bytes of the dominant kernel (per launch, or per step for workloads
    that launch it many times per step), from the committed rocprofv3 summary,
    if it was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{workload}_profile.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    m = re.search(r"kernel_sources_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_(?:launch|step):\s*([0-9]+)", text)
    if not m or not t or m.group(1) != kernel_hash(workload):
        return None
    return int(t.group(1))


# ----------------------------------------------------------------- workloads

class Workload:
    """Device buffers plus one step's launches; algorithmic bytes per step."""
    name = ""
    bytes_per_step = 0
    dominant = ""
    dominant_bytes = 0
    dtype = "f32"          # the arithmetic type of the step (fp32 accumulation); movement-only steps override

    def step(self, k):
        raise NotImplementedError

    def dominant_launch(self, k):
        """Launch only the dominant kernel of step k (for its per-launch timing)."""
        self.step(k)


class Layout:
    """Where the N rank buffers of a workload live in HBM.

    arena      (default) each rank owns one region of HBM (RankArena: regions a
               large power of two apart plus a stagger, 4 KiB unless the workload
               names its own); every buffer of rank r
               is carved from region r, as a real rank's buffers sit in its GPU
    staggered  one allocation per buffer set, ranks 4 KiB apart (gc_rank_buffers)
    separate   one torch allocation per rank buffer
    """

    def __init__(self, args, nranks, stagger=None):
        import collective_communication_reduction_amd as gc
        self.gc = gc
        self.kind = args.layout
        self.nranks = nranks
        self.stagger = args.stagger if args.stagger is not None else (stagger or 4096)
        self.arena = (gc.RankArena(nranks, region_bytes=getattr(args, "region_bytes", None), stagger_bytes=self.stagger,
                                   max_region=args.max_region << 30)
                      if self.kind == "arena" else None)

    def buffers(self, count, tdt):
        import torch
        if self.kind == "separate":
            return [torch.empty(count, dtype=tdt, device="cuda") for _ in range(self.nranks)]
        if self.kind == "staggered":
            return self.gc.gc_rank_buffers(self.nranks, count, tdt, stagger_bytes=self.stagger)
        return self.arena.alloc(count, tdt)

    def name(self):
        if self.kind == "separate":
            return "separate allocations"
        if self.kind == "staggered":
            return f"one allocation per buffer set, {self.stagger} B per-rank stagger"
        reg = self.arena.region
        size = f"{reg >> 30} GiB" if reg % (1 << 30) == 0 else f"{reg} B"
        return f"rank arena: {size} region per rank, {self.stagger} B stagger"


def _keyed(seed, r, stream=0):
    from gen.host import stream_key
    return stream_key(seed, r, stream)


class AllReduceWorkload(Workload):
    def __init__(self, args, nranks, count, dtype, op):
        import torch
        import collective_communication_reduction_amd as gc
        from gen import device as GD
        self.gc = gc
        self.N, self.S, self.dtype_storage, self.op = nranks, count, dtype, op
        tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
        es = 2 if dtype == "bf16" else 4
        self.algo = args.algo
        self.order = args.order
        self.name = (f"ar_{dtype}_n{nranks}" + ("" if self.algo == "fused" else "_rs_ag") +
                     ("" if self.order == "ring" else f"_{self.order}"))
        self.bytes_per_step = 2 * nranks * count * es          # the all-reduce's own bytes, either algorithm
        self.dominant = ("reduce_vec_kernel (fused all-reduce)" if self.algo == "fused" else
                         "reduce_vec_kernel (reduce-scatter to scratch) + gather_vec_kernel (all-gather)")
        self.dominant_bytes = self.bytes_per_step
        self.scratch = None
        if self.algo == "rs_ag":
            self.scratch = torch.empty(max(1, gc.gc_all_reduce_scratch_bytes(count, nranks, dtype, "rs_ag")),
                                       dtype=torch.uint8, device="cuda")
        self.sets = []
        L = Layout(args, nranks)
        self.layout = L.name()
        # enough replica sets that one rotation touches >= 1 GiB (4x the 256 MB MALL)
        reps = max(args.replicas, -(-(1 << 30) // self.bytes_per_step))
        for rep in range(reps):
            send = L.buffers(count, tdt)
            recv = L.buffers(count, tdt)
            for r, t in enumerate(send):
                if dtype == "bf16":
                    GD.fill_normal_bf16(t, _keyed(args.seed, r), 1e-3)
                else:
                    GD.fill_uniform_f32(t, _keyed(args.seed, r))
            self.sets.append((send, recv))
        # Pointer arrays marshalled once per replica set, and the stream fixed: for a
        # few-microsecond kernel the per-call marshalling would otherwise starve the GPU.
        self.ptrs = [(gc.gc_pointers(send), gc.gc_pointers(recv)) for send, recv in self.sets]
        self.stream = torch.cuda.current_stream().cuda_stream
        torch.cuda.synchronize()

    def step(self, k, stream=None):
        sp, rp = self.ptrs[k % len(self.ptrs)]
        self.gc.gc_all_reduce(sp, rp, op=self.op, order=self.order, algo=self.algo, scratch=self.scratch,
                              count=self.S, dtype=self.dtype_storage,
                              stream=self.stream if stream is None else stream)

    def config(self):
        return {"workload": self.name, "nranks": self.N, "count_per_rank": self.S, "storage": self.dtype_storage,
                "op": self.op, "order": self.order, "algo": self.algo, "replicas": len(self.sets), "layout": self.layout}

    def cpu_sample(self, seed):
        """Oracle all-reduce on the first quarter of every rank's buffer."""
        import numpy as np
        from gen import host as G
        from oracle import collectives as C
        S = self.S // 4
        xs = []
        for r in range(self.N):
            key = _keyed(seed, r)
            xs.append(G.normal_bf16(key, np.arange(S), 1e-3) if self.dtype_storage == "bf16" else
                      G.uniform_f32(key, np.arange(S)))
        es = 2 if self.dtype_storage == "bf16" else 4
        return (lambda: C.all_reduce(xs, self.dtype_storage, self.op, "ring"), 2 * self.N * S * es,
                f"oracle ring all-reduce of {self.N} ranks x {S} {self.dtype_storage} (first quarter of each buffer)")


class DdpWorkload(Workload):
    """Llama-7B gradient set, 8 ranks, 25 MiB buckets: pack -> fused all-reduce (avg) -> unpack per bucket,
    or (zero_copy) the bucket all-reduced in place over the gradient tensors, with the sum of squares
    of the synced gradients accumulated for norm clipping."""

    def __init__(self, args, zero_copy=False):
        import torch
        import collective_communication_reduction_amd as gc
        from gen import device as GD
        from gen.workloads import WORKLOADS, llama7b_tensors
        self.gc = gc
        cfg = WORKLOADS["ddp_llama7b"]
        self.N = cfg["nranks"]
        self.name = "ddp_llama7b"
        numels = [n for _, n in llama7b_tensors()]
        self.numels = numels
        self.plan = gc.BucketPlan(numels, "bf16", cfg["cap_bytes"], reverse=True)
        total = sum(numels)
        # one flat allocation per rank; tensor t is a view at its model-order offset
        L = Layout(args, self.N)
        self.flat = L.buffers(total, torch.bfloat16)
        self.layout = L.name()
        offs, run = [], 0
        for n in numels:
            offs.append(run)
            run += n
        for r in range(self.N):
            GD.fill_normal_bf16(self.flat[r], _keyed(args.seed, r), cfg["sigma"])
        self.tensors = [self.flat[r][o:o + n] for r in range(self.N) for o, n in zip(offs, numels)]
        self.tensor_ptrs = gc.gc_pointers(self.tensors)   # the gradients persist: marshal once
        big = max(self.plan.bucket_numel)
        self.bufs = [L.buffers(big, torch.bfloat16) for _ in range(2)] if not zero_copy else []
        self.bucket_bytes = [b * 2 for b in self.plan.bucket_numel]
        self.zero_copy = zero_copy
        if zero_copy:
            self.name = "ddp_llama7b_zero_copy"
            self.sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
            self.bytes_per_step = 2 * self.N * sum(self.bucket_bytes)
            self.dominant = "bucket_ar_kernel (zero-copy bucket all-reduce + sum of squares)"
        else:
            self.bytes_per_step = 6 * self.N * sum(self.bucket_bytes)
            self.dominant = "reduce_vec_kernel (fused all-reduce of each bucket)"
        self.dominant_bytes = 2 * self.N * sum(self.bucket_bytes)
        torch.cuda.synchronize()

    def step(self, k, marks=None):
        gc, plan, N = self.gc, self.plan, self.N
        if self.zero_copy:
            self.sumsq.zero_()
            for b in range(plan.nbuckets):
                plan.all_reduce(b, self.tensor_ptrs, N, op="avg", order="ring", sumsq=self.sumsq)
            return
        for b in range(plan.nbuckets):
            bufs = self.bufs[b & 1]
            n = plan.bucket_numel[b]
            views = [x[:n] for x in bufs]
            plan.pack(b, self.tensor_ptrs, views, N)
            if marks:
                marks[b][0].record()
            gc.gc_all_reduce(views, views, op="avg", order="ring", algo="fused")
            if marks:
                marks[b][1].record()
            plan.unpack(b, views, self.tensor_ptrs, N)

    def allreduce_in_step(self, steps):
        """ms per step inside the all-reduce launches, each bracketed by events within
        whole steps, so that every bucket is read right after its pack as in the timed
        steps (None for the zero-copy step, whose launches are the whole step).  Part of
        each freshly packed bucket is then served by the 256 MB MALL, so bytes over this
        time are algorithmic bytes, not HBM bytes."""
        import torch
        if self.zero_copy:
            return None
        marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(self.plan.nbuckets)]
        total = 0.0
        for k in range(steps):
            self.step(k, marks)
            torch.cuda.synchronize()
            total += sum(a.elapsed_time(b) for a, b in marks)
        return total / steps

    def dominant_launch(self, k):
        plan = self.plan
        if self.zero_copy:
            self.step(k)
            return
        for b in range(plan.nbuckets):
            views = [x[:plan.bucket_numel[b]] for x in self.bufs[b & 1]]
            self.gc.gc_all_reduce(views, views, op="avg", order="ring", algo="fused")

    def config(self):
        return {"workload": self.name, "nranks": self.N, "params": sum(self.numels), "storage": "bf16",
                "buckets": self.plan.nbuckets, "cap_bytes": 25 * 1024 * 1024, "op": "avg", "order": "ring",
                "zero_copy": self.zero_copy, "layout": self.layout,
                **({} if self.zero_copy else {
                    "cache_note": "each bucket is read by the all-reduce right after its pack, and part of it is "
                                  "then served by the 256 MB MALL: value counts algorithmic bytes, not HBM bytes"})}

    def cpu_sample(self, seed):
        import numpy as np
        from gen import host as G
        from oracle import buckets as OB
        from oracle import collectives as C
        b = 1  # [final_norm, L31 norms, L31 down_proj]: a mixed bucket
        ts = OB.assign_buckets(self.numels, 2, 25 * 1024 * 1024, reverse=True)[b]
        offs = np.cumsum([0] + self.numels)
        n_per = 1 << 20  # first 1 Mi elements of each tensor of the bucket
        numels = [min(self.numels[t], n_per) for t in ts]
        per_rank = []
        for r in range(self.N):
            key = _keyed(seed, r)
            per_rank.append([G.normal_bf16(key, offs[t] + np.arange(n), 1e-3) for t, n in zip(ts, numels)])
        idx = list(range(len(ts)))

        def run():
            flats = [OB.pack(per_rank[r], idx, numels) for r in range(self.N)]
            out = C.all_reduce(flats, "bf16", "avg", "ring")
            return [OB.unpack(out[r], idx, numels) for r in range(self.N)]
        nbytes = (2 if self.zero_copy else 6) * self.N * sum(numels) * 2
        return run, nbytes, f"oracle pack + ring all-reduce + unpack of bucket {b} truncated to {sum(numels)} elements"


class FsdpWorkload(Workload):
    """One transformer layer flattened, 64 ranks: reduce-scatter (avg) bf16 -> fp32, then all-gather bf16."""

    def __init__(self, args):
        import torch
        import collective_communication_reduction_amd as gc
        from gen import device as GD
        from gen.workloads import fsdp_layer_tensors
        self.gc = gc
        self.N = 64
        self.name = "fsdp_layer_n64"
        total = sum(n for _, n in fsdp_layer_tensors())
        self.S = -(-total // self.N) * self.N
        self.rc = self.S // self.N
        L = Layout(args, self.N)
        self.grads = L.buffers(self.S, torch.bfloat16)
        self.gshards = L.buffers(self.rc, torch.float32)
        self.pshards = L.buffers(self.rc, torch.bfloat16)
        self.params = L.buffers(self.S, torch.bfloat16)
        self.layout = L.name()
        for r in range(self.N):
            GD.fill_normal_bf16(self.grads[r], _keyed(args.seed, r, 0), 1e-3)
            GD.fill_normal_bf16(self.pshards[r], _keyed(args.seed, r, 1), 0.02)
        self.rs_bytes = self.N * self.S * 2 + self.N * self.rc * 4
        self.ag_bytes = self.N * self.rc * 2 + self.N * self.S * 2
        self.bytes_per_step = self.rs_bytes + self.ag_bytes
        self.dominant = "reduce_vec_kernel (reduce-scatter, 64 ranks)"
        self.dominant_bytes = self.rs_bytes
        torch.cuda.synchronize()

    def step(self, k):
        self.gc.gc_reduce_scatter(self.grads, self.gshards, op="avg", order="ring")
        self.gc.gc_all_gather(self.pshards, self.params)

    def dominant_launch(self, k):
        self.gc.gc_reduce_scatter(self.grads, self.gshards, op="avg", order="ring")

    def config(self):
        return {"workload": self.name, "nranks": self.N, "flat_numel": self.S, "shard": self.rc,
                "rs": "bf16->fp32 avg ring", "ag": "bf16", "layout": self.layout}

    def cpu_sample(self, seed):
        import numpy as np
        from gen import host as G
        from oracle import sampled as SM
        m = 1 << 17  # 131072 sampled outputs of owner 5

        vals = np.stack([G.normal_bf16(_keyed(seed, i, 0), 5 * self.rc + np.arange(m), 1e-3) for i in range(self.N)])

        def run():
            return SM.reduce_scatter_at(vals, np.full(m, 5), np.arange(m), self.rc, "bf16", "fp32", "avg", "ring")
        return run, self.N * m * 2 + m * 4, f"oracle reduce-scatter of {m} outputs of owner 5 (64-way fold each)"


class Fsdp2Workload(Workload):
    """The same layer as FSDP2 shards it, 64 ranks: every parameter its own dim-0 shard (DTensor Shard(0)),
    reduce-scatter (avg) bf16 -> fp32 and all-gather bf16 per parameter, one launch each."""

    def __init__(self, args):
        import numpy as np
        import torch
        import collective_communication_reduction_amd as gc
        from gen import device as GD
        from gen.workloads import fsdp_layer_shapes
        self.gc = gc
        self.N = N = 64
        self.name = "fsdp2_layer_n64"
        shapes = fsdp_layer_shapes()
        self.rows = [r for _, r, _ in shapes]
        self.cols = [c for _, _, c in shapes]
        P = len(shapes)
        numel = [r * c for r, c in zip(self.rows, self.cols)]
        offs = np.concatenate([[0], np.cumsum(numel)]).astype(np.int64)
        S = int(offs[-1])

        def shard(p, r):
            c = -(-self.rows[p] // N)
            return min(self.rows[p], r * c) * self.cols[p], min(self.rows[p], (r + 1) * c) * self.cols[p]
        soffs = [np.concatenate([[0], np.cumsum([shard(p, r)[1] - shard(p, r)[0] for p in range(P)])]).astype(np.int64)
                 for r in range(N)]
        most = max(int(x[-1]) for x in soffs)
        L = Layout(args, N)
        self.layout = L.name()
        grads = L.buffers(S, torch.bfloat16)
        gsh = L.buffers(most, torch.float32)
        psh = L.buffers(most, torch.bfloat16)
        params = L.buffers(S, torch.bfloat16)
        for r in range(N):
            GD.fill_normal_bf16(grads[r], _keyed(args.seed, r, 0), 1e-3)
            GD.fill_normal_bf16(psh[r], _keyed(args.seed, r, 1), 0.02)
        self.bufs = (grads, gsh, psh, params)

        def views(buf, o, r):
            return [buf[r][o[r][p] if isinstance(o, list) else o[p]:(o[r][p + 1] if isinstance(o, list) else o[p + 1])]
                    for p in range(P)]
        # the gradient, shard and parameter tensors persist across steps: marshal once
        self.g = gc.gc_pointers([t for r in range(N) for t in views(grads, offs, r)])
        self.gs = gc.gc_pointers([t for r in range(N) for t in views(gsh, soffs, r)])
        self.ps = gc.gc_pointers([t for r in range(N) for t in views(psh, soffs, r)])
        self.pa = gc.gc_pointers([t for r in range(N) for t in views(params, offs, r)])
        shard_elems = sum(int(x[-1]) for x in soffs)
        self.rs_bytes = N * S * 2 + shard_elems * 4
        self.ag_bytes = shard_elems * 2 + N * S * 2
        self.bytes_per_step = self.rs_bytes + self.ag_bytes
        self.S = S
        self.dominant = "reduce_vec_kernel (per-parameter reduce-scatter, 64 ranks; 9 launches)"
        self.dominant_bytes = self.rs_bytes
        torch.cuda.synchronize()

    def rs(self):
        self.gc.gc_fsdp2_reduce_scatter(self.g, self.gs, self.rows, self.cols, self.N, "bf16", "fp32", "avg", "ring")

    def step(self, k):
        self.rs()
        self.gc.gc_fsdp2_all_gather(self.ps, self.pa, self.rows, self.cols, self.N, "bf16")

    def dominant_launch(self, k):
        self.rs()

    def config(self):
        return {"workload": self.name, "nranks": self.N, "params": len(self.rows), "numel": self.S,
                "sharding": "per-parameter dim 0 (torch.chunk rule)", "rs": "bf16->fp32 avg ring", "ag": "bf16",
                "layout": self.layout}

    def cpu_sample(self, seed):
        import numpy as np
        from gen import host as G
        from oracle import fsdp2 as F2
        # q_proj's first 64 columns (the dim-0 shards of a column slice are those of the whole
        # parameter) and the two norm vectors, 64 ranks
        rows, cols = [4096, 4096, 4096], [64, 1, 1]
        n = [r * c for r, c in zip(rows, cols)]
        grads = [[G.normal_bf16(_keyed(seed, r, 0), np.arange(k, dtype=np.uint64) + 1000 * p, 1e-3)
                  for p, k in enumerate(n)] for r in range(self.N)]

        def run():
            return F2.reduce_scatter(grads, rows, cols, "bf16", "fp32", "avg", "ring")
        nbytes = self.N * sum(n) * 2 + sum(n) * 4
        return run, nbytes, "oracle per-parameter ring reduce-scatter of 64 ranks x (q_proj[:, :64] + 2 x 4096) bf16"


class HierWorkload(Workload):
    """Two-level all-reduce, 16 ranks as 2 groups of 8 (two nodes of eight GPUs), 64 MiB bf16 each, avg."""

    def __init__(self, args):
        import torch
        import collective_communication_reduction_amd as gc
        from gen import device as GD
        from gen.workloads import WORKLOADS
        self.gc = gc
        cfg = WORKLOADS["hier_ar_n16"]
        self.cfg = cfg
        self.N, self.S, self.count = cfg["nranks"], cfg["group"], cfg["count"]
        self.name = "hier_ar_n16"
        L = Layout(args, self.N, stagger=cfg.get("stagger"))
        self.layout = L.name()
        self.send = L.buffers(self.count, torch.bfloat16)
        self.recv = L.buffers(self.count, torch.bfloat16)
        for r in range(self.N):
            GD.fill_normal_bf16(self.send[r], _keyed(args.seed, r), cfg["sigma"])
        self.sp, self.rp = gc.gc_pointers(self.send), gc.gc_pointers(self.recv)
        self.bytes_per_step = 2 * self.N * self.count * 2
        self.dominant = "hier_vec_kernel (fused two-level all-reduce)"
        self.dominant_bytes = self.bytes_per_step
        torch.cuda.synchronize()

    def step(self, k):
        self.gc.gc_hier_all_reduce(self.sp, self.rp, self.S, op="avg", order="ring", count=self.count,
                                   dtype="bf16")

    def config(self):
        return {"workload": self.name, "nranks": self.N, "groups": self.N // self.S, "group_size": self.S,
                "count_per_rank": self.count, "storage": "bf16", "op": "avg", "order": "ring (two-level)",
                "layout": self.layout}

    def cpu_sample(self, seed):
        import numpy as np
        from gen import host as G
        from oracle import hierarchical as H
        m = 1 << 21  # the first 2,097,152 elements of each rank
        xs = [G.normal_bf16(_keyed(seed, r), np.arange(m, dtype=np.uint64), self.cfg["sigma"]) for r in range(self.N)]

        def run():
            return H.all_reduce(xs, self.S, "bf16", "avg", "ring")
        return run, 2 * self.N * m * 2, f"oracle three-ring two-level all-reduce of 16 ranks x {m} bf16"


class HsdpWorkload(Workload):
    """HSDP step of one transformer layer on 16 ranks as 2 groups of 8 (two nodes of eight GPUs): the gradient
    reduce-scatter (avg, bf16 -> fp32) over all 16 ranks, member i of every group keeping shard i, then the
    all-gather of the bf16 parameter shards inside each group."""

    def __init__(self, args):
        import torch
        import collective_communication_reduction_amd as gc
        from gen import device as GD
        from gen.workloads import WORKLOADS, fsdp_layer_tensors
        self.gc = gc
        cfg = WORKLOADS["hsdp_layer_n16"]
        self.N, self.G = cfg["nranks"], cfg["group"]
        self.R = self.N // self.G
        self.name = "hsdp_layer_n16"
        total = sum(n for _, n in fsdp_layer_tensors())
        self.S = -(-total // self.G) * self.G
        self.rc = self.S // self.G
        L = Layout(args, self.N, stagger=cfg.get("stagger"))
        self.grads = L.buffers(self.S, torch.bfloat16)
        self.gshards = L.buffers(self.rc, torch.float32)
        self.pshards = L.buffers(self.rc, torch.bfloat16)
        self.params = L.buffers(self.S, torch.bfloat16)
        self.layout = L.name()
        for r in range(self.N):
            GD.fill_normal_bf16(self.grads[r], _keyed(args.seed, r, 0), cfg["grad_sigma"])
            GD.fill_normal_bf16(self.pshards[r], _keyed(args.seed, r % self.G, 1), 0.02)
        self.gp, self.sp = gc.gc_pointers(self.grads), gc.gc_pointers(self.gshards)
        groups = [range(g * self.G, (g + 1) * self.G) for g in range(self.R)]
        self.agp = [(gc.gc_pointers([self.pshards[r] for r in m]), gc.gc_pointers([self.params[r] for r in m]))
                    for m in groups]
        self.rs_bytes = self.N * self.S * 2 + self.N * self.rc * 4
        self.ag_bytes = self.N * self.rc * 2 + self.N * self.S * 2
        self.bytes_per_step = self.rs_bytes + self.ag_bytes
        self.dominant = "hier_vec_kernel (HSDP reduce-scatter, 2 x 8 ranks)"
        self.dominant_bytes = self.rs_bytes
        torch.cuda.synchronize()

    def rs(self):
        self.gc.gc_hsdp_reduce_scatter(self.gp, self.sp, self.G, op="avg", order="ring", recv_count=self.rc,
                                       in_dtype="bf16", out_dtype="fp32")

    def step(self, k):
        self.rs()
        for pin, pout in self.agp:
            self.gc.gc_all_gather(pin, pout, count=self.rc, dtype="bf16")

    def dominant_launch(self, k):
        self.rs()

    def config(self):
        return {"workload": self.name, "nranks": self.N, "groups": self.R, "group_size": self.G,
                "flat_numel": self.S, "shard": self.rc, "rs": "bf16->fp32 avg, two-level ring",
                "ag": "bf16 inside each group", "layout": self.layout}

    def cpu_sample(self, seed):
        import numpy as np
        from gen import host as G
        from oracle import sampled as SM
        m, i = 1 << 16, 3                     # 65536 sampled outputs of member 3 (every group holds them)
        p = i * self.rc + np.arange(m)
        vals = np.stack([G.normal_bf16(_keyed(seed, r, 0), p, 1e-3) for r in range(self.N)])

        def run():
            g0, m0 = SM.hier_fold_starts(p, self.S, self.G, self.R, "ring", chunk=self.rc)
            return SM.hier_reduce_positions(vals, self.G, g0, m0, "bf16", "avg", "fp32")
        return run, self.N * m * 2 + m * 4, f"oracle two-level fold of {m} outputs of member {i} (16-way each)"


class MoeWorkload(Workload):
    """MoE dispatch all-to-all, 8 ranks x 16384 tokens x 4096 bf16, top-2 of 64 experts, Zipf(1.1)."""

    def __init__(self, args):
        import numpy as np
        import torch
        import collective_communication_reduction_amd as gc
        from gen import device as GD
        from gen.workloads import WORKLOADS, moe_send_layout
        self.gc = gc
        cfg = WORKLOADS["moe_a2a_n8"]
        self.N, self.H = cfg["nranks"], cfg["hidden"]
        self.name = "moe_a2a_n8"
        self.splits, rows = moe_send_layout(args.seed, self.N, cfg["tokens"], cfg["experts"], cfg["topk"],
                                            cfg["zipf_s"])
        self.row_bytes = self.H * 2
        L = Layout(args, self.N)
        self.layout = L.name()
        recv_rows = self.splits.sum(axis=(0, 2))
        # every rank's buffer sized for the largest rank, at the same offset of each rank's memory
        send_full = L.buffers(max(len(r) for r in rows) * self.H, torch.bfloat16)
        recv_full = L.buffers(int(recv_rows.max()) * self.H, torch.bfloat16)
        self.send = [send_full[s][:len(rows[s]) * self.H] for s in range(self.N)]
        self.recv = [recv_full[d][:int(recv_rows[d]) * self.H] for d in range(self.N)]
        for s in range(self.N):
            GD.fill_normal_bf16_rows(self.send[s], torch.from_numpy(rows[s]).cuda(), self.H, _keyed(args.seed, s), 1.0)
        total_rows = int(self.splits.sum())
        self.bytes_per_step = 2 * total_rows * self.row_bytes
        self.dominant = "segment_vec_kernel (all-to-all, one contiguous copy per block)"
        self.dominant_bytes = self.bytes_per_step
        self.frac_dst0 = float(self.splits[:, 0, :].sum() / total_rows)
        self.rows = rows
        self.dtype = "bf16"   # pure movement of bf16 rows
        torch.cuda.synchronize()

    def step(self, k):
        self.gc.gc_all_to_all(self.send, self.recv, self.splits, self.row_bytes)

    def config(self):
        return {"workload": self.name, "nranks": self.N, "tokens": 16384, "hidden": self.H, "experts": 64,
                "topk": 2, "zipf_s": 1.1, "rows": int(self.splits.sum()), "frac_rows_to_rank0": round(self.frac_dst0, 4),
                "layout": self.layout}

    def cpu_sample(self, seed):
        import numpy as np
        from gen import host as G
        from oracle import collectives as C
        # the full routing, with 64-element rows (the first 64 of the 4096 hidden values)
        h = 64
        cols = np.arange(h, dtype=np.uint64)
        sends = [G.normal_bf16(_keyed(seed, s), (self.rows[s].astype(np.uint64)[:, None] * np.uint64(self.H)
                                                 + cols).reshape(-1), 1.0) for s in range(self.N)]
        sub = self.splits

        def run():
            return C.all_to_all(sends, sub, h)
        return run, 2 * int(sub.sum()) * h * 2, "oracle all-to-all of every row, 64 of 4096 columns"


class MoeEpWorkload(Workload):
    """Expert-parallel MoE data flow, 8 ranks x 16384 tokens x 4096 bf16, top-2 of 64 experts, Zipf(1.1):
    routing plan on the device, dispatch from token order, combine with the gate weights back to
    token order.  The experts are the identity (their compute is not part of the data flow), so the
    combine reads the dispatched rows."""

    def __init__(self, args):
        import numpy as np
        import torch
        import collective_communication_reduction_amd as gc
        from gen import device as GD
        from gen.workloads import WORKLOADS, route_tokens
        self.gc = gc
        cfg = WORKLOADS["moe_ep_n8"]
        self.cfg = cfg
        N, T, H, K = cfg["nranks"], cfg["tokens"], cfg["hidden"], cfg["topk"]
        self.N, self.T, self.H, self.K, self.E = N, T, H, K, cfg["experts"] // N
        self.name = "moe_ep_n8"
        self.seed = args.seed
        self.experts_host = [route_tokens(args.seed, s, T, cfg["experts"], K, cfg["zipf_s"]) for s in range(N)]
        self.experts = [torch.from_numpy(e.reshape(-1).astype(np.int32)).cuda() for e in self.experts_host]
        self.ntok = [T] * N
        self.weights = [torch.empty(T * K, dtype=torch.float32, device="cuda") for _ in range(N)]
        for s in range(N):
            GD.fill_uniform_f32(self.weights[s], _keyed(args.seed, s, 3))
        L = Layout(args, N)
        self.layout = L.name()
        self.tokens = L.buffers(T * H, torch.bfloat16)
        for s in range(N):
            GD.fill_normal_bf16(self.tokens[s], _keyed(args.seed, s), 1.0)
        self.splits = torch.empty(N * N * self.E, dtype=torch.int64, device="cuda")
        self.dest = [torch.empty(T * K * 2, dtype=torch.int32, device="cuda") for _ in range(N)]
        self.scratch = torch.empty(gc.gc_moe_route_scratch_bytes(self.ntok, K, self.E), dtype=torch.uint8,
                                   device="cuda")
        # the receive buffers are sized from one routing plan (a real step reads the splits back too)
        gc.gc_moe_route(self.experts, self.ntok, K, self.E, self.splits, self.dest, self.scratch)
        self.recv_rows = [int(x) for x in self.splits.view(N, N, self.E).sum(dim=(0, 2)).cpu()]
        recv_full = L.buffers(max(self.recv_rows) * H, torch.bfloat16)
        self.recv = [recv_full[d][:self.recv_rows[d] * H] for d in range(N)]
        self.out = L.buffers(T * H, torch.bfloat16)
        self.row_bytes = H * 2
        routes = N * T * K
        self.route_bytes = routes * (4 + 8) + N * N * self.E * 8
        self.dispatch_bytes = N * T * self.row_bytes + routes * (self.row_bytes + 8)
        self.combine_bytes = routes * (self.row_bytes + 8 + 4) + N * T * self.row_bytes
        self.bytes_per_step = self.route_bytes + self.dispatch_bytes + self.combine_bytes
        self.dominant = "combine_kernel (inverse all-to-all + weighted un-permute)"
        self.dominant_bytes = self.combine_bytes
        self.frac_dst0 = self.recv_rows[0] / routes
        torch.cuda.synchronize()

    def route(self):
        self.gc.gc_moe_route(self.experts, self.ntok, self.K, self.E, self.splits, self.dest, self.scratch)

    def dispatch(self):
        self.gc.gc_moe_dispatch(self.tokens, self.ntok, self.dest, self.K, self.row_bytes, self.recv,
                                self.recv_rows)

    def combine(self):
        self.gc.gc_moe_combine(self.recv, self.recv_rows, self.dest, self.weights, self.ntok, self.K, self.H,
                               "bf16", self.out)

    def step(self, k):
        self.route()
        self.dispatch()
        self.combine()

    def dominant_launch(self, k):
        self.combine()

    def config(self):
        c = self.cfg
        return {"workload": self.name, "nranks": self.N, "tokens": self.T, "hidden": self.H,
                "experts": c["experts"], "topk": self.K, "zipf_s": c["zipf_s"], "storage": "bf16",
                "frac_rows_to_rank0": round(self.frac_dst0, 4), "experts_compute": "identity",
                "layout": self.layout}

    def cpu_sample(self, seed):
        import numpy as np
        from gen import host as G
        from oracle import moe as OM
        # the first 4096 tokens of every source, 1024 of the 4096 hidden values
        t, h, K = 4096, 1024, self.K
        ex = [e[:t] for e in self.experts_host]
        idx = (np.arange(t, dtype=np.uint64)[:, None] * np.uint64(self.H) + np.arange(h, dtype=np.uint64)).reshape(-1)
        toks = [G.normal_bf16(_keyed(seed, s), idx, 1.0) for s in range(self.N)]
        w = [G.uniform_f32(_keyed(seed, s, 3), np.arange(t * K, dtype=np.uint64)).reshape(t, K)
             for s in range(self.N)]

        def run():
            recv = OM.dispatch(toks, ex, self.N, self.E, h)
            return OM.combine(recv, ex, w, self.N, self.E, h, "bf16")
        routes = self.N * t * K
        nbytes = routes * 12 + self.N * t * h * 2 + routes * (h * 2 + 8) + routes * (h * 2 + 12) + self.N * t * h * 2
        return run, nbytes, (f"oracle routing plan + dispatch + combine of the first {t} tokens of each source, "
                             f"the first {h} of {self.H} hidden values")


def make(args):
    if args.workload in ("ar_bf16_n8", "ar_fp32_n4"):
        from gen.workloads import WORKLOADS
        c = WORKLOADS[args.workload]
        return AllReduceWorkload(args, c["nranks"], c["count"], c["dtype"], c["op"])
    if args.workload == "ddp_llama7b":
        return DdpWorkload(args)
    if args.workload == "ddp_llama7b_zero_copy":
        return DdpWorkload(args, zero_copy=True)
    if args.workload == "fsdp_layer_n64":
        return FsdpWorkload(args)
    if args.workload == "moe_ep_n8":
        return MoeEpWorkload(args)
    if args.workload == "fsdp2_layer_n64":
        return Fsdp2Workload(args)
    if args.workload == "hier_ar_n16":
        return HierWorkload(args)
    if args.workload == "hsdp_layer_n16":
        return HsdpWorkload(args)
    return MoeWorkload(args)


# ----------------------------------------------------------------- timing

def time_steps(fn, steps, warmup, per_step=None):
    """HIP events on torch's current stream (the stream every libgc launch uses).
    Returns ms per step over the whole timed region; with per_step (a list), also
    appends each step's own event time."""
    import torch
    for k in range(warmup):
        fn(k)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps)] if per_step is not None else None
    start.record()
    for k in range(steps):
        fn(warmup + k)
        if marks:
            marks[k].record()
    stop.record()
    torch.cuda.synchronize()
    if marks:
        prev = start
        for m in marks:
            per_step.append(prev.elapsed_time(m))
            prev = m
    return start.elapsed_time(stop) / steps  # ms per step


def copy_ceiling(nbytes=2 << 30, steps=10):
    """A plain 16-byte copy of nbytes through libgc's segment-copy kernel (a
    one-rank, one-block all-to-all): read + write bytes per second, GB/s."""
    import torch
    import collective_communication_reduction_amd as gc
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    splits = [[[1]]]

    def run(_k):
        gc.gc_all_to_all([a], [b], splits, nbytes)
    ms = time_steps(run, steps, 2)
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def host_cpu():
    """CPU model name and the number of hardware threads of this host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


def cpu_baseline(w, seed, budget_s=10.0):
    run, nbytes, what = w.cpu_sample(seed)
    run()  # warm the code paths once (numpy allocations)
    t0 = time.perf_counter()
    reps = 0
    while True:  # about budget_s of single-threaded oracle work
        run()
        reps += 1
        if time.perf_counter() - t0 >= budget_s or reps >= 1000:
            break
    per = (time.perf_counter() - t0) / reps
    model, threads = host_cpu()
    return {"value": round(nbytes / per / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{what}; {reps} runs, {per:.3g} s each, single-threaded numpy",
            "host_cpu": model, "host_threads": threads}


def _quantile(xs, q):
    ys = sorted(xs)
    if not ys:
        return 0.0
    k = (len(ys) - 1) * q
    lo = int(k)
    hi = min(lo + 1, len(ys) - 1)
    return ys[lo] + (ys[hi] - ys[lo]) * (k - lo)


def measure(w, steps, warmup):
    """The step time (K steps back to back), the per-step spread (the same K steps,
    each bracketed by its own events: for a few-microsecond step those records are
    host work the GPU would wait for, so they stay out of the first pass), and the
    dominant kernel's time per step: the whole step where it is one launch, else
    its launches alone."""
    ms = time_steps(w.step, steps, warmup)
    step_ms = []
    time_steps(w.step, steps, 0, step_ms)
    kms = ms if type(w).dominant_launch is Workload.dominant_launch else \
        time_steps(w.dominant_launch, max(3, steps // 5), 2)
    return ms, step_ms, kms


def roofline(w, kms):
    achieved = w.dominant_bytes / (kms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profiles(w.name),
            "kernel": w.dominant, "algorithmic_bytes_per_launch": w.dominant_bytes}


def graph_us(launch, n):
    """GPU time per launch of `launch(k, stream)` for k < n, captured into one HIP
    graph and replayed (no host work between launches: the device-side cost of
    each launch)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for k in range(n):                 # warm the code path on a side stream
            launch(k, s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        for k in range(n):
            launch(k, cs)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    reps = 20
    start.record()
    for _ in range(reps):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) * 1e3 / (reps * n)


def launch_floor(w):
    """The all-reduce call path at its smallest: the same ranks and type, 4 elements
    per rank (one element per owner chunk, N workgroups), back to back eagerly and
    in a HIP graph.  The difference between a workload's time and this floor is
    what its bytes cost beyond launching."""
    import torch
    gc = w.gc
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[w.dtype_storage]
    send = [torch.ones(4, dtype=tdt, device="cuda") for _ in range(w.N)]
    recv = [torch.empty(4, dtype=tdt, device="cuda") for _ in range(w.N)]
    sp, rp = gc.gc_pointers(send), gc.gc_pointers(recv)
    stream = torch.cuda.current_stream().cuda_stream

    def one(_k, st):
        gc.gc_all_reduce(sp, rp, op=w.op, order="ring", count=4, dtype=w.dtype_storage, stream=st)
    eager = time_steps(lambda k: one(k, stream), 200, 20) * 1e3
    empty = graph_us(lambda _k, _st: torch.cuda._sleep(0), 100)   # a kernel that does nothing
    return {"eager_us": round(eager, 3), "graph_us": round(graph_us(one, 100), 3),
            "empty_kernel_graph_us": round(empty, 3),
            "what": f"all-reduce of 4 elements per rank ({w.N} ranks, {w.dtype_storage}, {w.N} workgroups); "
                    "empty kernel: torch.cuda._sleep(0)"}


def extra_line(w, steps, warmup):
    """ms per step, value and roofline of one more workload, for the default run's extra keys."""
    ms, step_ms, kms = measure(w, steps, warmup)
    out = {"ms_per_step": round(ms, 5), "value": round(w.bytes_per_step / (ms * 1e-3) / 1e9, 2),
           "unit": "GB/s (algorithmic bytes per step / step time)", "dtype": w.dtype, "steps": steps,
           "warmup": warmup, "bytes_per_step": w.bytes_per_step,
           "step_ms": {"median": round(_quantile(step_ms, 0.5), 5), "min": round(min(step_ms), 5),
                       "p90": round(_quantile(step_ms, 0.9), 5)},
           "roofline": roofline(w, kms), "config": w.config()}
    return out


EXTRAS = (
    # (key, workload, layout, steps, warmup): at least 50 timed steps after 5 warm-up steps, except the
    # 7B DDP passes (about 0.1 s each), which are timed over 3 full passes
    ("ar_bf16_n8_separate", "ar_bf16_n8", "separate", 50, 10),
    ("ar_fp32_n4", "ar_fp32_n4", "arena", 50, 10),
    ("fsdp_layer_n64", "fsdp_layer_n64", "arena", 50, 5),
    ("moe_a2a_n8", "moe_a2a_n8", "arena", 50, 10),
    ("ddp_llama7b", "ddp_llama7b", "arena", 3, 1),
    # the rows past the target's configurations, one workload each
    ("ddp_llama7b_zero_copy", "ddp_llama7b_zero_copy", "arena", 3, 1),
    ("moe_ep_n8", "moe_ep_n8", "arena", 50, 10),
    ("fsdp2_layer_n64", "fsdp2_layer_n64", "arena", 50, 5),
    ("hier_ar_n16", "hier_ar_n16", "arena", 50, 10),
    ("hsdp_layer_n16", "hsdp_layer_n16", "arena", 50, 5),
)


def run_extras(args):
    """The remaining configurations of the target, measured one after another in
    this process (each one's memory released before the next is built)."""
    import gc as pygc
    import torch
    out = {}
    pats = Patterns.optional()
    for key, name, layout, steps, warmup in EXTRAS:
        a = argparse.Namespace(**vars(args))
        a.workload, a.layout, a.algo, a.order, a.stagger = name, layout, "fused", "ring", None
        w = make(a)
        line = extra_line(w, steps, warmup)
        if name == "ar_fp32_n4":
            # A 7-microsecond step is shorter than one pass of the Python loop that issues it, so the
            # eager steps measure the host.  In a HIP graph (one replay = 128 launches over the 32
            # replica sets) the launches run back to back on the device: that is the kernel's time.
            floor = launch_floor(w)
            n = len(w.ptrs)
            g_us = graph_us(w.step, 4 * n)
            line["graph"] = {"us_per_step": round(g_us, 3), "value": round(w.bytes_per_step / (g_us * 1e-6) / 1e9, 2),
                             "launches_per_replay": 4 * n}
            line["roofline"] = roofline(w, g_us * 1e-3)
            line["roofline"]["note"] = "per-launch time in a HIP graph (the eager steps are bound by the host loop)"
            line["launch_floor"] = floor
            line["over_floor_us"] = round(g_us - floor["graph_us"], 3)
        if name == "ddp_llama7b":
            ar = w.allreduce_in_step(steps)
            line["allreduce_in_step"] = {
                "ms_per_step": round(ar, 4), "value": round(w.dominant_bytes / (ar * 1e-3) / 1e9, 2),
                "unit": "GB/s (algorithmic: part of each freshly packed bucket is served by the 256 MB MALL)"}
            line["roofline"]["note"] = "the 226 bucket all-reduces launched alone (no pack before them): HBM-bound"
        side = pats.beside(w) if pats is not None else None
        if side is not None:
            line["pattern"] = side
        if not args.no_cpu and layout == "arena":
            # the oracle beside each workload, on a bounded sample (about 3 s of work each)
            line["cpu_baseline"] = cpu_baseline(w, args.seed, budget_s=3.0)
        out[key] = line
        del w
        pygc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


class Patterns:
    """The access-pattern kernels of bench_patterns.hip (libbenchpatterns.so): unordered
    kernels that move the same bytes as a collective, in the same tiles, with no fold
    order and no floating point, so that a kernel can be timed beside the pattern of its
    own reads and writes on the same buffers."""

    def __init__(self):
        import ctypes
        import torch
        import collective_communication_reduction_amd as gc
        path = os.path.join(ROOT, "libbenchpatterns.so")
        if not os.path.exists(path):
            raise RuntimeError("libbenchpatterns.so is missing: run __graft_entry__.build() first")
        self.gc = gc
        self.lib = ctypes.CDLL(path)
        VPP = ctypes.POINTER(ctypes.c_void_p)
        self.lib.bp_pattern.restype = ctypes.c_int
        self.lib.bp_pattern.argtypes = [VPP, ctypes.c_int, VPP, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        self.sink = torch.zeros(256, dtype=torch.int32, device="cuda")
        self.stream = torch.cuda.current_stream().cuda_stream

    @classmethod
    def optional(cls):
        """The pattern kernels for the bench line's `pattern` keys, or None (with a note) if they are not
        built: the keys are context, the measurement does not depend on them."""
        if not os.path.exists(os.path.join(ROOT, "libbenchpatterns.so")):
            print("libbenchpatterns.so is not built: the bench line carries no pattern keys", file=sys.stderr)
            return None
        return cls()

    def pattern(self, sets, nvec, chunk_vecs=0, mode=0, out_mult=1):
        """A launch of the pattern over sets, a list of (sources, destinations) tensor lists rotated over the steps."""
        gc = self.gc
        ptrs = [(gc.gc_pointers(s) if s else None, gc.gc_pointers(d) if d else None, len(s), len(d))
                for s, d in sets]

        def run(k):
            sp, dp, ns, nd = ptrs[k % len(ptrs)]
            rc = self.lib.bp_pattern(sp, ns, dp, nd, nvec, chunk_vecs, mode, out_mult, self.sink.data_ptr(),
                                     self.stream)
            if rc != 0:
                raise RuntimeError(f"bp_pattern returned {rc}")
        return run

    def entries(self, w):
        """(name, launch, bytes per launch) of a workload's dominant kernel, its pattern and the pattern's
        reads alone; None for workloads without a contiguous twin."""
        if isinstance(w, AllReduceWorkload) and w.algo == "fused":
            nv = w.S * (2 if w.dtype_storage == "bf16" else 4) // 16
            return [("library fused all-reduce", w.step, w.bytes_per_step),
                    (f"pattern {w.N} in : {w.N} out", self.pattern(w.sets, nv), w.bytes_per_step),
                    (f"pattern {w.N} in, no stores", self.pattern([(s, []) for s, _ in w.sets], nv),
                     w.bytes_per_step // 2)]
        if isinstance(w, HierWorkload):
            nv = w.count * 2 // 16
            return [("library two-level all-reduce", w.step, w.bytes_per_step),
                    ("pattern 16 in : 16 out", self.pattern([(w.send, w.recv)], nv), w.bytes_per_step),
                    ("pattern 16 in, no stores", self.pattern([(w.send, [])], nv), w.bytes_per_step // 2)]
        if isinstance(w, FsdpWorkload):
            nv, cv = w.S * 2 // 16, w.rc * 2 // 16
            return [("library reduce-scatter bf16 -> fp32", w.dominant_launch, w.rs_bytes),
                    ("pattern 64 in : owner's 2x out", self.pattern([(w.grads, w.gshards)], nv, cv, 1, 2), w.rs_bytes),
                    ("pattern 64 in, no stores", self.pattern([(w.grads, [])], nv), w.N * w.S * 2)]
        if isinstance(w, HsdpWorkload):
            nv, cv = w.S * 2 // 16, w.rc * 2 // 16
            return [("library HSDP reduce-scatter bf16 -> fp32", lambda _k: w.rs(), w.rs_bytes),
                    ("pattern 16 in : both holders' 2x out", self.pattern([(w.grads, w.gshards)], nv, cv, 1, 2),
                     w.rs_bytes),
                    ("pattern 16 in, no stores", self.pattern([(w.grads, [])], nv), w.N * w.S * 2)]
        return None

    @staticmethod
    def compare(label, entries, rounds=3, steps=20, warm=3):
        """Time every entry, alternating over rounds; medians with min and max."""
        import statistics
        rates = {name: [] for name, _, _ in entries}
        for _ in range(rounds):
            for name, fn, nbytes in entries:
                ms = time_steps(fn, steps, warm)
                rates[name].append(nbytes / (ms * 1e-3) / 1e9)
        out = {"case": label, "rows": []}
        for name, _, nbytes in entries:
            r = rates[name]
            med = statistics.median(r)
            out["rows"].append({"kernel": name, "GBps": round(med, 1), "min": round(min(r), 1),
                                "max": round(max(r), 1), "us": round(nbytes / med / 1e3, 1), "bytes": nbytes})
        return out

    def beside(self, w):
        """The short form for the bench line: the dominant kernel and its pattern on the same buffers
        (2 alternating rounds of 10 launches), or None."""
        e = self.entries(w)
        if e is None or e[0][2] < (1 << 28):    # a few-microsecond launch times the host loop, not the kernel
            return None
        c = self.compare(w.name, e[:2], rounds=2, steps=10, warm=2)
        lib_r, pat_r = c["rows"]
        return {"pattern": pat_r["kernel"], "pattern_GBps": pat_r["GBps"], "kernel_GBps": lib_r["GBps"],
                "frac_of_pattern": round(lib_r["GBps"] / pat_r["GBps"], 4),
                "what": "the dominant kernel and an unordered kernel moving the same bytes in the same tiles "
                        "(bench_patterns.hip), timed alternately on the same buffers"}


def run_patterns(args):
    """Each dominant kernel against the access-pattern kernels on the same buffers, in
    one process, alternating over rounds: the gap between the two is what the kernel
    itself costs.  Also reads alone, writes alone and a 1 : 1 copy on two 2 GiB buffers."""
    import gc as pygc
    import torch
    P = Patterns()
    gc = P.gc

    def release():
        pygc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    def ns(**kw):
        a = argparse.Namespace(**vars(args))
        a.algo, a.order, a.stagger, a.layout = "fused", "ring", None, "arena"
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    results = []
    # plain streams on two 2 GiB buffers
    n = 2 << 30
    a_ = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b_ = torch.empty(n, dtype=torch.uint8, device="cuda")
    nvec = n // 16

    def lib_copy(_k):
        gc.gc_all_to_all([a_], [b_], [[[1]]], n)
    results.append(P.compare("2 GiB streams (one allocation each)", [
        ("library segment copy (device-scope stores)", lib_copy, 2 * n),
        ("pattern copy 1 in : 1 out", P.pattern([([a_], [b_])], nvec), 2 * n),
        ("pattern reads alone", P.pattern([([a_], [])], nvec), n),
        ("pattern writes alone", P.pattern([([], [b_])], nvec), n)]))
    print(json.dumps(results[-1]), flush=True)
    del a_, b_
    release()

    for name, layout in (("ar_bf16_n8", "arena"), ("ar_bf16_n8", "separate"), ("hier_ar_n16", "arena"),
                         ("fsdp_layer_n64", "arena"), ("hsdp_layer_n16", "arena")):
        w = make(ns(workload=name, layout=layout))
        label = f"{name} ({w.layout})" if name.startswith(("ar_", "hier")) else f"{name} reduce-scatter ({w.layout})"
        results.append(P.compare(label, P.entries(w)))
        print(json.dumps(results[-1]), flush=True)
        del w
        release()
    print(json.dumps({"patterns": results, "rounds": 3, "steps": 20, "warmup": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library runs all N ranks as buffers in one MI355X's HBM "
              f"(no collectives across GPUs), so --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.init()
    if args.patterns:
        run_patterns(args)
        return
    w = make(args)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
    # The measurement: K steps back to back, nothing else inside the timed region.
    ms, step_ms, kms = measure(w, args.steps, args.warmup)
    value = w.bytes_per_step / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC if w.name == "ar_bf16_n8" else
        f"algorithmic GB/s (bytes the step must move / step time) for {w.name} on 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": w.config(),
        "roofline": roofline(w, kms),
        "bytes_per_step": w.bytes_per_step,
        "step_ms": {"median": round(_quantile(step_ms, 0.5), 5), "min": round(min(step_ms), 5),
                    "p90": round(_quantile(step_ms, 0.9), 5)},
    }
    if hasattr(w, "allreduce_in_step"):
        ar = w.allreduce_in_step(max(3, args.steps // 5))
        if ar is not None:
            out["allreduce_in_step"] = {
                "ms_per_step": round(ar, 4), "value": round(w.dominant_bytes / (ar * 1e-3) / 1e9, 2),
                "unit": "GB/s (algorithmic: part of each freshly packed bucket is served by the 256 MB MALL)"}
    pats = Patterns.optional() if not args.no_extras else None
    if pats is not None:
        side = pats.beside(w)
        if side is not None:
            out["pattern"] = side
    if not args.no_extras and isinstance(w, AllReduceWorkload):
        # the same steps captured in one HIP graph and replayed: the kernel back to back with no
        # host work between launches (the eager loop adds the launch gap to every step)
        n = 4 * len(w.ptrs)
        g_us = graph_us(w.step, n)
        out["graph"] = {"us_per_step": round(g_us, 3), "value": round(w.bytes_per_step / (g_us * 1e-6) / 1e9, 2),
                        "launches_per_replay": n}
    if not args.no_copy_ceiling:
        ceiling = copy_ceiling()
        out["copy_ceiling"] = {"value": round(ceiling, 2), "unit": "GB/s",
                               "kernel": "segment_vec_kernel, one 2 GiB block (16-byte loads, 16-byte device-scope stores)",
                               "frac": round(out["roofline"]["achieved"] / ceiling, 4)}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, args.seed)
    else:
        out["cpu_baseline"] = None
    if not args.no_extras and args.workload == "ar_bf16_n8":
        del w
        import gc as pygc
        pygc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out.update(run_extras(args))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
