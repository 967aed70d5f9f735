"""Work counts and reporting arithmetic of the benchmark (no part of the method).

FLOP conventions: the backward does five products per unmasked (query, key)
pair -- the recomputed scores Q K^T, dP = dO V^T, dV += P^T dO, dK += dS^T Q,
dQ += dS K -- each 2*d FLOP, so 10*d FLOP per pair.  Only unmasked pairs of
kept blocks count (masked halves of diagonal tiles do not).  The forward does
two products, 4*d FLOP per unmasked pair.
"""
import numpy as np

__all__ = ["pairs_dense", "bwd_flops_dense", "fwd_flops", "bwd_flops_kept", "amdahl",
           "MI355X_PEAK"]

# Published MI355X peaks (dense, no sparsity), per second.
MI355X_PEAK = {"bf16_flops": 2.5e15, "hbm_bytes": 8.0e12, "fp32_flops": 157.3e12,
               "fp64_flops": 78.6e12}


def pairs_dense(N, causal):
    return N * (N + 1) // 2 if causal else N * N


def bwd_flops_dense(B, Hq, N, d, causal):
    return 10 * B * Hq * d * pairs_dense(N, causal)


def fwd_flops(B, Hq, N, d, causal):
    return 4 * B * Hq * d * pairs_dense(N, causal)


def bwd_flops_kept(keep, N, d, block, causal):
    """keep: [..., nqb] boolean (or block weights, nonzero = kept)."""
    keep = np.asarray(keep) != 0
    idx = np.nonzero(keep)[-1].astype(np.int64)
    rows = np.minimum(block, N - idx * block)  # the last block may be partial
    if causal:
        pairs = rows * (idx * block) + rows * (rows + 1) // 2
    else:
        pairs = rows * N
    return int(10 * d * pairs.sum())


def amdahl(total, part, speedup):
    """Whole-job time and gain when only `part` of `total` runs `speedup` x faster."""
    new = (total - part) + part / speedup
    return new, total / new, total / (total - part) if total > part else float("inf")
