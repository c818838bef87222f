"""MoE expert-parallel data flow around the all-to-all (test infrastructure only).

DTLM §8 ("专家并行和 MoE 通信") gives the layer's data flow: the router picks
top-k experts per token, tokens are packed by target expert / rank, an
All-to-All dispatches them, the local experts compute, an All-to-All combines
the results back, and the outputs are restored to token order.  The router
and the experts need weights and are out of scope; the data movement around
them is what this module defines, as compositions of `collectives.all_to_all`:

  route_plan   routing (global expert of each (token, k)) -> splits and, for
               every (token, k), the destination rank and row of its copy.
               Send order at a source: by global expert (= destination rank,
               then local expert), then by token; the receive layout is
               all_to_all's (local expert, source, sent order).
  dispatch     pack the tokens' rows in send order, then all_to_all.
  combine      the inverse: for every source token, its k expert rows come back
               and are combined as sum_k w_k * y_k.  Arithmetic (a reading: the
               pages give none): rows widened to fp32, each product w_k * y_k
               rounded to fp32, the products added in k order starting from
               k = 0, the sum rounded to the row type (bf16: nearest-even).

Dropped routes (a reading: the pages name a capacity limit that drops tokens
but no format for it): an expert id outside [0, N * E) marks a route that is
not sent.  It is not counted in the splits, its destination is (-1, -1),
dispatch copies nothing for it and combine leaves it out of the sum (the fold
starts at the first route kept); a token with no route kept gets zeros.
"""

import numpy as np

from .collectives import _widen, a2a_recv_offsets, all_to_all
from .numerics import f32_to_bf16


def route_plan(experts, nranks, experts_per_rank):
    """experts[s]: int array [T, K] of global expert ids of source s's tokens.

    Returns (splits int64 [N][N][E], dest_rank list of int64 [T*K], dest_row list
    of int64 [T*K]); entry t*K + k describes the copy of token t for its k-th
    expert.  Rows go to rank g // E, local expert g % E.
    """
    N, E = nranks, experts_per_rank
    splits = np.zeros((N, N, E), dtype=np.int64)
    orders = []
    for s in range(N):
        ex = np.asarray(experts[s], dtype=np.int64)
        T, K = ex.shape
        g = ex.reshape(-1)
        tok = np.repeat(np.arange(T), K)
        keep = (g >= 0) & (g < N * E)
        order = np.lexsort((tok, g))          # send order: by global expert, then token
        orders.append(order[keep[order]])
        counts = np.bincount(g[keep], minlength=N * E)
        splits[s] = counts.reshape(N, E)
    roff = a2a_recv_offsets(splits)
    dest_rank, dest_row = [], []
    for s in range(N):
        ex = np.asarray(experts[s], dtype=np.int64)
        g = ex.reshape(-1)
        dr = np.full(len(g), -1, dtype=np.int64)
        dw = np.full(len(g), -1, dtype=np.int64)
        seen = {}
        for idx in orders[s]:                 # walk the send order; rows of one (s, g) block keep it
            ge = int(g[idx])
            d, e = ge // E, ge % E
            k = seen.get(ge, 0)
            seen[ge] = k + 1
            dr[idx] = d
            dw[idx] = roff[s, d, e] + k
        dest_rank.append(dr)
        dest_row.append(dw)
    return splits, dest_rank, dest_row


def dispatch(tokens, experts, nranks, experts_per_rank, hidden):
    """tokens[s]: flat [T*hidden] rows of source s.  Returns the receive buffers (flat)."""
    splits, _, _ = route_plan(experts, nranks, experts_per_rank)
    sends = []
    for s in range(nranks):
        ex = np.asarray(experts[s], dtype=np.int64)
        T, K = ex.shape
        tok = np.repeat(np.arange(T), K)
        g = ex.reshape(-1)
        order = np.lexsort((tok, g))
        order = order[(g[order] >= 0) & (g[order] < nranks * experts_per_rank)]
        rows = np.asarray(tokens[s]).reshape(T, hidden)
        sends.append(rows[tok[order]].reshape(-1))
    return all_to_all(sends, splits, hidden)


def combine_rows(y, w, dtype, keep=None):
    """The weighted sum of one or more tokens' K expert rows.

    y: [K, n, H] rows in storage type (bf16 as bit patterns), w: fp32 [n, K],
    keep: optional bool [n, K] (False: a dropped route, left out).
    Returns [n, H] in `dtype`: widen to fp32, p_k = fp32(w_k * y_k), then
    ((p_0 + p_1) + p_2) + ... in fp32 over the kept routes, then round to the
    row type; zeros where no route is kept."""
    y = np.asarray(y)
    w = np.asarray(w, dtype=np.float32)
    K, n, H = y.shape
    keep = np.ones((n, K), dtype=bool) if keep is None else np.asarray(keep, dtype=bool)
    acc = np.zeros((n, H), dtype=np.float32)
    started = np.zeros(n, dtype=bool)
    with np.errstate(over="ignore", invalid="ignore"):
        for k in range(K):
            yk = _widen(y[k].reshape(-1), dtype).reshape(n, H)
            term = (w[:, k:k + 1] * yk).astype(np.float32)
            summed = (acc + term).astype(np.float32)
            kk = keep[:, k]
            acc = np.where((kk & started)[:, None], summed, np.where(kk[:, None], term, acc))
            started |= kk
    return f32_to_bf16(acc) if dtype == "bf16" else acc.astype(np.float32)


def combine(expert_out, experts, weights, nranks, experts_per_rank, hidden, dtype):
    """expert_out[d]: flat rows in rank d's receive layout; weights[s]: fp32 [T, K].
    Returns per source the token-major combined rows (flat), in `dtype`.
    Row (t, k) of source s is fetched from rank dest_rank, row dest_row: the
    inverse all-to-all (transposed splits) followed by the un-permute."""
    _, dest_rank, dest_row = route_plan(experts, nranks, experts_per_rank)
    outs = []
    for s in range(nranks):
        w = np.asarray(weights[s], dtype=np.float32)
        T, K = w.shape
        y = np.zeros((K, T, hidden), dtype=np.asarray(expert_out[0]).dtype)
        keep = np.zeros((T, K), dtype=bool)
        for k in range(K):
            for t in range(T):
                d, r = int(dest_rank[s][t * K + k]), int(dest_row[s][t * K + k])
                if d < 0:
                    continue
                keep[t, k] = True
                y[k, t] = np.asarray(expert_out[d])[r * hidden:(r + 1) * hidden]
        outs.append(combine_rows(y, w, dtype, keep).reshape(-1))
    return outs
