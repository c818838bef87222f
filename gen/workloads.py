"""Shapes and synthetic-input recipes of the gradient-sync workloads.

Shapes only, plus the MoE routing draw (an input: which expert each token is
sent to).  No collective arithmetic and no bucket layout live here.

  ar_fp32_n4      all-reduce (sum), 4 ranks x 1,048,576 fp32, uniform(-1,1)
  ar_bf16_n8      all-reduce (avg), 8 ranks x 33,554,432 bf16 (64 MiB), normal(0,1e-3)
  ddp_llama7b     DDP bucketed all-reduce (avg) of a Llama-7B-shaped gradient set,
                  8 ranks, bf16 normal(0,1e-3), 25 MiB buckets filled in reverse
  fsdp_layer_n64  FSDP unit step on one transformer layer (202,383,360 params),
                  64 ranks: reduce-scatter (avg) bf16 -> fp32 shards, then
                  all-gather of bf16 parameter shards normal(0,0.02)
  fsdp2_layer_n64 the same layer with per-parameter dim-0 shards (FSDP2)
  hier_ar_n16     two-level all-reduce (avg), 16 ranks in groups of 8,
                  33,554,432 bf16 each, normal(0,1e-3)
  hsdp_layer_n16  HSDP step on the layer: 16 ranks in groups of 8, gradient
                  reduce-scatter (avg) bf16 -> fp32 over all 16 ranks with member
                  i of each group keeping shard i, then all-gather in each group
  moe_a2a_n8      MoE dispatch all-to-all, 8 ranks x 16384 tokens x 4096 bf16
                  normal(0,1), top-2 of 64 experts (8 per rank), Zipf(1.1)
  moe_ep_n8       the same tokens and routing through route -> dispatch -> combine

Key of rank r's data in every workload: stream_key(seed, r, stream).
"""

import numpy as np

from .host import MASK64, mix64, stream_key, u64

VOCAB, HIDDEN, MLP, LAYERS = 32000, 4096, 11008, 32

LAYER_TENSORS = (
    ("q_proj", HIDDEN * HIDDEN), ("k_proj", HIDDEN * HIDDEN), ("v_proj", HIDDEN * HIDDEN),
    ("o_proj", HIDDEN * HIDDEN), ("gate_proj", MLP * HIDDEN), ("up_proj", MLP * HIDDEN),
    ("down_proj", HIDDEN * MLP), ("attn_norm", HIDDEN), ("mlp_norm", HIDDEN),
)


def llama7b_tensors():
    """(name, numel) in model definition order: embedding, 32 layers, final norm, LM head."""
    out = [("embed_tokens", VOCAB * HIDDEN)]
    for layer in range(LAYERS):
        out += [(f"layers.{layer}.{n}", k) for n, k in LAYER_TENSORS]
    out += [("final_norm", HIDDEN), ("lm_head", VOCAB * HIDDEN)]
    return out


def fsdp_layer_tensors():
    """One transformer layer's parameters in definition order (the FSDP unit)."""
    return list(LAYER_TENSORS)


def fsdp_layer_shapes():
    """(name, rows, cols) of the layer's parameters: Linear weights are [out, in], norms [hidden] (one column)."""
    shapes = {"q_proj": (HIDDEN, HIDDEN), "k_proj": (HIDDEN, HIDDEN), "v_proj": (HIDDEN, HIDDEN),
              "o_proj": (HIDDEN, HIDDEN), "gate_proj": (MLP, HIDDEN), "up_proj": (MLP, HIDDEN),
              "down_proj": (HIDDEN, MLP), "attn_norm": (HIDDEN, 1), "mlp_norm": (HIDDEN, 1)}
    return [(n, *shapes[n]) for n, _ in LAYER_TENSORS]


WORKLOADS = {
    "ar_fp32_n4": dict(nranks=4, count=1_048_576, dtype="fp32", op="sum", dist="uniform"),
    "ar_bf16_n8": dict(nranks=8, count=33_554_432, dtype="bf16", op="avg", dist="normal", sigma=1e-3),
    "ddp_llama7b": dict(nranks=8, dtype="bf16", op="avg", dist="normal", sigma=1e-3,
                        cap_bytes=25 * 1024 * 1024),
    "fsdp_layer_n64": dict(nranks=64, dtype="bf16", grad_sigma=1e-3, param_sigma=0.02),
    "fsdp2_layer_n64": dict(nranks=64, dtype="bf16", grad_sigma=1e-3, param_sigma=0.02),
    # 64 KiB between consecutive ranks' regions: measured 6.31 TB/s against 6.04 with 4 KiB for this
    # 16-rank layout (8- and 64-rank layouts keep 4 KiB: 64 KiB was equal or up to 2.7 % slower there)
    "hier_ar_n16": dict(nranks=16, group=8, count=33_554_432, dtype="bf16", op="avg", sigma=1e-3,
                        stagger=65536),
    # the same 64 KiB stagger (6.12 TB/s against 5.98 with 4 KiB for this step; 16 KiB measured equal)
    "hsdp_layer_n16": dict(nranks=16, group=8, dtype="bf16", grad_sigma=1e-3, stagger=65536),
    "moe_a2a_n8": dict(nranks=8, tokens=16384, hidden=4096, experts=64, topk=2, zipf_s=1.1),
    "moe_ep_n8": dict(nranks=8, tokens=16384, hidden=4096, experts=64, topk=2, zipf_s=1.1, dtype="bf16"),
}


# ------------------------------------------------------------------ MoE routing

def zipf_cdf(n_experts, s):
    """Cumulative P(e) with P(e) proportional to (e+1)^-s, e = 0..n_experts-1 (double)."""
    w = np.array([(e + 1.0) ** (-s) for e in range(n_experts)], dtype=np.float64)
    return np.cumsum(w) / w.sum()


def _route_draw(key, token, j):
    """The j-th uniform double in [0,1) of a token: U64(64*token + j//4, j%4) >> 11, times 2**-53."""
    idx = np.asarray(token, dtype=np.uint64) * np.uint64(64) + np.uint64(j // 4)
    return (u64(key, idx, j % 4) >> np.uint64(11)).astype(np.float64) * 2.0 ** -53


def route_tokens(seed, rank, tokens, n_experts, topk, s, stream=2):
    """Top-k distinct experts per token; expert k>1 redrawn until distinct (at most 256 draws)."""
    key = stream_key(seed, rank, stream)
    cdf = zipf_cdf(n_experts, s)
    t = np.arange(tokens, dtype=np.int64)
    chosen = np.full((tokens, topk), -1, dtype=np.int64)
    draw = 0
    for slot in range(topk):
        pending = np.ones(tokens, dtype=bool)
        while pending.any():
            if draw >= 256:
                raise RuntimeError("routing redraw budget exhausted")
            u = _route_draw(key, t, draw)
            e = np.searchsorted(cdf, u, side="right")
            e = np.minimum(e, n_experts - 1)
            dup = np.zeros(tokens, dtype=bool)
            for prev in range(slot):
                dup |= chosen[:, prev] == e
            take = pending & ~dup
            chosen[take, slot] = e[take]
            pending &= ~take
            draw += 1
    return chosen


def moe_send_layout(seed, nranks, tokens, n_experts, topk, s):
    """Routing of every source rank, as splits[src][dst][local_expert] and per-source row tokens.

    Each (token, chosen expert) pair is one row.  Rank s's send rows are ordered
    by global expert (= destination rank, then local expert), then by token.
    Returns (splits int64 [N][N][E], rows: list of int32 arrays of token ids).
    """
    E = n_experts // nranks
    splits = np.zeros((nranks, nranks, E), dtype=np.int64)
    rows = []
    for src in range(nranks):
        chosen = route_tokens(seed, src, tokens, n_experts, topk, s)
        tok = np.repeat(np.arange(tokens, dtype=np.int64), topk)
        exp = chosen.reshape(-1)
        order = np.lexsort((tok, exp))
        rows.append(tok[order].astype(np.int32))
        counts = np.bincount(exp, minlength=n_experts)
        splits[src] = counts.reshape(nranks, E)
    return splits, rows


__all__ = ["WORKLOADS", "llama7b_tensors", "fsdp_layer_tensors", "fsdp_layer_shapes", "zipf_cdf", "route_tokens",
           "moe_send_layout", "stream_key", "mix64", "MASK64"]
