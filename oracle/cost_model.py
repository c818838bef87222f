"""The pages' analytic communication estimates (context numbers; test infrastructure only).

alpha-beta model (AIG6 §6.1.4; NXMR §2.3): one message of M bytes costs
alpha + M / B.  A ring all-reduce over N ranks of an S-byte buffer sends
2(N-1)/N * S bytes per rank in 2(N-1) steps (DTLM §2 "All-Reduce"; NXMR §2.2),
so T = 2(N-1) * alpha + 2(N-1)/N * S / B.  The naive reduce-to-root then
broadcast sends 2(N-1) * S (NXMR §2.2).
"""


def ring_allreduce_bytes_per_rank(S, N):
    return 2.0 * (N - 1) / N * S


def ring_rs_or_ag_bytes_per_rank(S, N):
    return (N - 1) / N * S


def naive_allreduce_bytes(S, N):
    return 2.0 * (N - 1) * S


def ring_allreduce_time(S, N, alpha_s, bw_bytes_per_s):
    return 2 * (N - 1) * alpha_s + ring_allreduce_bytes_per_rank(S, N) / bw_bytes_per_s


def tp_allreduce_bytes_per_step(batch, seq_len, hidden, dtype_bytes, tp, layers, allreduces_per_layer=4):
    """Per-GPU ring traffic of tensor-parallel all-reduces in one step (NXMR §3.2-§3.3)."""
    message = batch * seq_len * hidden * dtype_bytes
    return ring_allreduce_bytes_per_rank(message, tp) * allreduces_per_layer * layers
