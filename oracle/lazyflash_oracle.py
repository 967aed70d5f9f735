"""Plain fp64 CPU oracle for LazyFlash-style attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library.

What it computes, and the passages it follows (the LazyFlash journal entry on
gyom.fr, "LazyFlash allège la rétropropagation de l'attention, 5,72 fois"):

* Forward: exact softmax attention, the same function FlashAttention computes
  (section "Le passage arrière fait deux fois le travail du passage avant": the
  forward is left exactly dense; the FlashAttention course page on voce.life,
  section "Le mécanisme": FlashAttention only reorganises memory traffic and
  stays exact).  Saves O and the natural-log logsumexp of each score row.
* Dense backward: the softmax-attention gradient written out with the row
  term D = rowsum(dO * O).
* Block masses: squared Frobenius norm of dO over each query block (section
  "Un budget sur la masse de gradient, et un tirage qui garde le gradient non
  biaisé": blocks are ranked by the norm of their output gradient).
* Budget tau: the discarded expected mass sum_b (1 - p_b) m_b equals
  delta * sum_b m_b, with p_b = min(1, m_b / tau), per (batch, head) (same
  section: the budget bounds the discarded share of gradient mass and adapts
  per head and per step).
* Draw and weights: keep block b with probability p_b, weight 1/p_b so the
  gradient is unbiased in expectation (same section).
* Sparse backward: skipped blocks contribute nothing and are never touched;
  kept blocks contribute their dense terms times w_b.
* Other selection rules, compared with the budget at equal backward time
  (section "Le choix des blocs pèse plus que la quantité sautée"): a fixed
  fraction of blocks chosen once for the whole run, where the budget adapts;
  and top-k, which removes the same blocks at every step, where the budget's
  draw changes from step to step.

Readings where the pages are silent (all listed in the design notes):
* tau is the unique root of the budget equation for 0 < delta < 1 (the
  literal "smallest tau" degenerates to tau -> 0, which keeps everything);
  delta = 0 gives tau = smallest positive mass, so every positive block has
  p = 1; an all-zero head gives tau = +inf and keeps nothing.
* Masses are summed in fp64 over the row-major flattening of the block with
  the fixed halving tree (x <- x[:L/2] + x[L/2:] until one value remains).
* The uniform of block (b, h, i) is (x0 >> 11) * 2**-53, x0 the first word of
  Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11) with key (seed, 0) and
  counter (i, h, b, 0); keep <=> u < p; w = fp32(fp64(1 / p)).
* A head whose masses are not all finite keeps every block with w = 1 and
  tau = NaN, so non-finite values propagate as in the dense backward.
* Grouped-query attention: query head h reads key/value head h // (Hq / Hkv).
* Fixed fraction f in (0, 1]: the budget's draw (p_b = min(1, m_b / tau),
  w = 1/p) with tau set so that the expected number of kept blocks,
  sum_b p_b, is c = f * n, n the number of positive-mass blocks.
* Top-k with fraction f in (0, 1]: keep the k = ceil(f * n) positive-mass
  blocks of largest mass (ties: lower block index first), weight 1, no draw;
  tau reports the smallest kept mass.
"""
import math

import numpy as np

__all__ = [
    "attn_fwd", "attn_fwd_rows", "attn_bwd_dense", "attn_bwd_sparse",
    "halving_tree_sum", "block_masses", "budget_discarded", "solve_tau",
    "philox4x64_10", "block_uniform", "select",
    "RULE_BUDGET", "RULE_FRACTION", "RULE_TOPK", "expected_kept", "solve_tau_fraction",
    "topk_keep", "select_rule",
]

RULE_BUDGET, RULE_FRACTION, RULE_TOPK = 0, 1, 2

MASK64 = (1 << 64) - 1


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------
def attn_fwd_rows(qh, kg, vg, scale, causal, rows):
    """O and logsumexp of the given query rows of one head.

    qh: [N, d] float64, kg, vg: [N, d] float64, rows: 1-D int array.
    Each row's softmax is independent of the others, so computing a subset of
    rows is the definition applied to those rows.
    Returns (o [len(rows), d], lse [len(rows)]).
    """
    rows = np.asarray(rows)
    s = scale * (qh[rows] @ kg.T)
    if causal:
        keys = np.arange(kg.shape[0])
        s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
    mx = s.max(axis=1)
    lse = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))
    p = np.exp(s - lse[:, None])
    return p @ vg, lse


def attn_fwd(q, k, v, scale, causal):
    """Exact attention forward: q [B,Hq,N,d], k, v [B,Hkv,N,d] (float64).

    Returns o [B,Hq,N,d] and lse [B,Hq,N] (natural log).
    """
    B, Hq, N, _ = q.shape
    G = Hq // k.shape[1]
    o = np.empty_like(q)
    lse = np.empty((B, Hq, N))
    rows = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            o[b, h], lse[b, h] = attn_fwd_rows(q[b, h], k[b, h // G], v[b, h // G],
                                               scale, causal, rows)
    return o, lse


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def _row_grads(qh, kg, vg, doh_rows, o_rows, lse_rows, scale, causal, rows):
    """Gradient terms of a set of query rows of one head.

    Returns (dq_rows, dk_part, dv_part): dq of the rows, and the parts of dK
    and dV [N, d] that those rows contribute.
    """
    s = scale * (qh[rows] @ kg.T)
    if causal:
        keys = np.arange(kg.shape[0])
        s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
    p = np.exp(s - lse_rows[:, None])
    d_row = (doh_rows * o_rows).sum(axis=1)          # D = rowsum(dO * O)
    dp = doh_rows @ vg.T                               # dP = dO V^T
    ds = p * (dp - d_row[:, None])                     # dS = P * (dP - D)
    dq = scale * (ds @ kg)                             # dQ = scale dS K
    dk = scale * (ds.T @ qh[rows])                     # dK = scale dS^T Q
    dv = p.T @ doh_rows                                # dV = P^T dO
    return dq, dk, dv


def attn_bwd_dense(q, k, v, dout, scale, causal, o=None, lse=None):
    """Dense attention backward in float64.  Returns dq, dk, dv.

    o / lse default to this module's own exact forward.
    """
    if o is None or lse is None:
        o, lse = attn_fwd(q, k, v, scale, causal)
    B, Hq, N, _ = q.shape
    G = Hq // k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rows = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            dqr, dkp, dvp = _row_grads(q[b, h], k[b, g], v[b, g], dout[b, h], o[b, h],
                                       lse[b, h], scale, causal, rows)
            dq[b, h] = dqr
            dk[b, g] += dkp
            dv[b, g] += dvp
    return dq, dk, dv


def attn_bwd_sparse(q, k, v, dout, block, keep, w, scale, causal,
                    heads=None, o=None, lse=None):
    """Block-sparse backward: kept query blocks only, each weighted by w.

    keep [B,Hq,nqb] bool, w [B,Hq,nqb] float.  Skipped blocks are never read and
    their dq rows are exact zeros.  ``heads`` restricts the work to a list of
    (b, h) pairs (every other output stays zero), which is how large shapes
    are checked one head group at a time.  o / lse default to this module's
    own exact forward on the rows needed.
    Returns dq, dk, dv in float64.
    """
    B, Hq, N, _ = q.shape
    G = Hq // k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in heads:
        g = h // G
        for i in np.nonzero(keep[b, h])[0]:
            rows = np.arange(i * block, min((i + 1) * block, N))
            if o is None or lse is None:
                o_rows, lse_rows = attn_fwd_rows(q[b, h], k[b, g], v[b, g], scale, causal, rows)
            else:
                o_rows, lse_rows = o[b, h, rows], lse[b, h, rows]
            dqr, dkp, dvp = _row_grads(q[b, h], k[b, g], v[b, g], dout[b, h, rows], o_rows,
                                       lse_rows, scale, causal, rows)
            wi = float(w[b, h, i])
            dq[b, h, rows] = wi * dqr
            dk[b, g] += wi * dkp
            dv[b, g] += wi * dvp
    return dq, dk, dv


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------
def halving_tree_sum(x):
    """Sum of a power-of-two-length float64 vector by the fixed halving tree.

    At every level the first half is added to the second half element-wise
    (x[k] + x[k + L/2]); the single value left is the sum.  Each addition is
    one IEEE double rounding, in this fixed order.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if n & (n - 1):
        raise ValueError("length must be a power of two")
    while n > 1:
        n //= 2
        x = x[..., :n] + x[..., n:]
    return x[..., 0]


def block_masses(dout, block):
    """m[b,h,i] = squared Frobenius norm of dO over query block i, in float64.

    dout [B,H,N,d] holds the exact values the kernel sees (bf16 or fp32
    upcast).  Their squares are exact in float64, so only the additions round,
    in halving-tree order over the row-major flattening of the block.  When N
    is not a multiple of block the last block has N - (nqb - 1) block rows; the
    tree runs over the full block*d slots with the missing rows as zeros
    (adding an exact zero changes nothing).
    """
    B, H, N, d = dout.shape
    nqb = -(-N // block)
    x = np.zeros((B, H, nqb * block, d))
    x[:, :, :N] = np.asarray(dout, dtype=np.float64)
    return halving_tree_sum((x * x).reshape(B, H, nqb, block * d))


def budget_discarded(m, tau):
    """f(tau) = sum_b (1 - p_b) m_b with p_b = min(1, m_b / tau) (exact-ish)."""
    m = np.asarray(m, dtype=np.float64)
    p = np.minimum(1.0, m / tau)
    return float(np.sum((1.0 - p) * m))


def solve_tau(m, delta):
    """tau of one (batch, head) for budget delta (0 <= delta < 1).

    On [m_(k), m_(k+1)] the discarded mass is A_k - Q_k / tau, where A_k and
    Q_k are the running sums of the k smallest positive masses and of their
    squares.  The first interval whose right end already meets the budget
    holds the root tau = Q_k / (A_k - delta * S).  Sums run sequentially in
    ascending order with one rounding per operation (no fused multiply-add).
    Returns +inf when no mass is positive, NaN when a mass is not finite.
    """
    m = np.asarray(m, dtype=np.float64)
    if not np.all(np.isfinite(m)):
        return math.nan
    pos = np.sort(m[m > 0.0])
    n = pos.shape[0]
    if n == 0:
        return math.inf
    if delta == 0.0:
        return float(pos[0])
    a = 0.0
    for x in pos:                      # S = A_n, ascending sequential sum
        a = a + float(x)
    target = delta * a
    a = 0.0
    qs = 0.0
    for k in range(n):
        mk = float(pos[k])
        a = a + mk
        qs = qs + mk * mk              # two roundings: product, then sum
        hi = float(pos[k + 1]) if k + 1 < n else math.inf
        if a - qs / hi >= target:
            return qs / (a - target)
    raise AssertionError("unreachable for delta < 1")


def philox4x64_10(counter, key):
    """Philox4x64 with 10 rounds (Salmon et al., SC'11), on Python integers.

    counter: 4 words, key: 2 words.  One round multiplies word 0 and word 2 by
    the two round multipliers, and forms (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2),
    hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key gains the two Weyl increments
    before every round but the first.
    """
    m0, m1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
    w0, w1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B
    c = [int(x) & MASK64 for x in counter]
    k0, k1 = int(key[0]) & MASK64, int(key[1]) & MASK64
    for r in range(10):
        if r:
            k0 = (k0 + w0) & MASK64
            k1 = (k1 + w1) & MASK64
        p0 = m0 * c[0]
        p1 = m1 * c[2]
        c = [((p1 >> 64) ^ c[1] ^ k0) & MASK64, p1 & MASK64,
             ((p0 >> 64) ^ c[3] ^ k1) & MASK64, p0 & MASK64]
    return c


def block_uniform(seed, b, h, i):
    """Uniform in [0, 1) of query block i of head h, batch b: 53 high bits."""
    x0 = philox4x64_10((i, h, b, 0), (seed, 0))[0]
    return (x0 >> 11) * 2.0 ** -53


def select(mass, delta, seed, b0=0):
    """Keep set and weights from masses [B,H,nqb] for budget delta and seed.

    Returns a dict with tau [B,H] float64, p, u [B,H,nqb] float64,
    keep [B,H,nqb] bool, w [B,H,nqb] float32 (0 when skipped),
    kept_idx [B,H,nqb] int32 (ascending, -1 padded), kept_count [B,H] int32.
    b0 is the batch index of mass[0] in the draw's counter (sequence b0 + b of
    a variable-length batch is drawn as batch entry b0 + b).
    """
    if not (0.0 <= delta < 1.0):
        raise ValueError("delta must be in [0, 1)")
    mass = np.asarray(mass, dtype=np.float64)
    B, H, nqb = mass.shape
    tau = np.empty((B, H))
    p = np.zeros((B, H, nqb))
    u = np.empty((B, H, nqb))
    keep = np.zeros((B, H, nqb), dtype=bool)
    w = np.zeros((B, H, nqb), dtype=np.float32)
    kept_idx = np.full((B, H, nqb), -1, dtype=np.int32)
    kept_count = np.zeros((B, H), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            t = solve_tau(mass[b, h], delta)
            tau[b, h] = t
            for i in range(nqb):
                u[b, h, i] = block_uniform(seed, b0 + b, h, i)
                mi = float(mass[b, h, i])
                if math.isnan(t):                       # non-finite head: dense
                    pi = 1.0
                elif mi == 0.0:
                    pi = 0.0
                else:
                    pi = min(1.0, mi / t)
                p[b, h, i] = pi
                if u[b, h, i] < pi:
                    keep[b, h, i] = True
                    w[b, h, i] = np.float32(1.0 / pi)
            idx = np.nonzero(keep[b, h])[0]
            kept_idx[b, h, :idx.size] = idx
            kept_count[b, h] = idx.size
    return dict(tau=tau, p=p, u=u, keep=keep, w=w, kept_idx=kept_idx, kept_count=kept_count)


# --------------------------------------------------------------------------
# other selection rules (section "Le choix des blocs pèse plus que la
# quantité sautée")
# --------------------------------------------------------------------------
def expected_kept(m, tau):
    """g(tau) = sum_b min(1, m_b / tau) over the positive masses."""
    m = np.asarray(m, dtype=np.float64)
    pos = m[m > 0.0]
    return float(np.sum(np.minimum(1.0, pos / tau)))


def solve_tau_fraction(m, f):
    """tau of one (batch, head) for a fixed expected kept fraction f in (0, 1].

    With the positive masses sorted ascending, m_(1) <= ... <= m_(n), and tau in
    [m_(k), m_(k+1)], the k smallest have p = m / tau and the others p = 1, so
    g(tau) = (n - k) + A_k / tau with A_k the running sum of the k smallest.
    g falls as tau grows; the first interval whose right end already has
    g <= c = f n holds the root tau = A_k / (c - (n - k)).  Sums run
    sequentially in ascending order, one rounding per operation.  c >= n
    keeps every positive block (tau = smallest positive mass); no positive
    mass gives +inf; a non-finite mass gives NaN.
    """
    if not (0.0 < f <= 1.0):
        raise ValueError("fraction must be in (0, 1]")
    m = np.asarray(m, dtype=np.float64)
    if not np.all(np.isfinite(m)):
        return math.nan
    pos = np.sort(m[m > 0.0])
    n = pos.shape[0]
    if n == 0:
        return math.inf
    c = f * float(n)
    if c >= float(n):
        return float(pos[0])
    a = 0.0
    for k in range(n):               # k + 1 smallest masses below tau
        a = a + float(pos[k])
        hi = float(pos[k + 1]) if k + 1 < n else math.inf
        sat = float(n - k - 1)       # blocks at p = 1
        if sat + a / hi <= c:
            return a / (c - sat)
    raise AssertionError("unreachable for 0 < c < n")


def topk_keep(m, f):
    """Keep mask of top-k for one (batch, head): the k = ceil(f n) positive
    masses of largest value, ties to the lower block index."""
    if not (0.0 < f <= 1.0):
        raise ValueError("fraction must be in (0, 1]")
    m = np.asarray(m, dtype=np.float64)
    keep = np.zeros(m.shape[0], dtype=bool)
    pos = np.nonzero(m > 0.0)[0]
    k = min(pos.size, math.ceil(f * float(pos.size)))
    order = sorted(pos.tolist(), key=lambda i: (-float(m[i]), i))
    keep[order[:k]] = True
    return keep


def select_rule(mass, rule, param, seed, b0=0):
    """Keep set and weights from masses [B,H,nqb] for one of the rules:
    RULE_BUDGET (param = delta, as select), RULE_FRACTION (param = f, the
    budget's draw with tau from solve_tau_fraction) or RULE_TOPK (param = f,
    deterministic, weight 1).  Same fields and b0 as select."""
    if rule == RULE_BUDGET:
        return select(mass, param, seed, b0)
    if rule not in (RULE_FRACTION, RULE_TOPK):
        raise ValueError("unknown rule")
    if not (0.0 < param <= 1.0):
        raise ValueError("fraction must be in (0, 1]")
    mass = np.asarray(mass, dtype=np.float64)
    B, H, nqb = mass.shape
    tau = np.empty((B, H))
    p = np.zeros((B, H, nqb))
    u = np.zeros((B, H, nqb))
    keep = np.zeros((B, H, nqb), dtype=bool)
    w = np.zeros((B, H, nqb), dtype=np.float32)
    kept_idx = np.full((B, H, nqb), -1, dtype=np.int32)
    kept_count = np.zeros((B, H), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            mh = mass[b, h]
            if not np.all(np.isfinite(mh)):          # non-finite head: dense
                tau[b, h] = math.nan
                p[b, h] = 1.0
                keep[b, h] = True
                w[b, h] = 1.0
            elif rule == RULE_TOPK:
                kk = topk_keep(mh, param)
                keep[b, h] = kk
                p[b, h] = kk.astype(np.float64)
                w[b, h] = np.where(kk, np.float32(1.0), np.float32(0.0))
                tau[b, h] = float(mh[kk].min()) if kk.any() else math.inf
            else:
                t = solve_tau_fraction(mh, param)
                tau[b, h] = t
                for i in range(nqb):
                    u[b, h, i] = block_uniform(seed, b0 + b, h, i)
                    mi = float(mh[i])
                    pi = 0.0 if mi == 0.0 else min(1.0, mi / t)
                    p[b, h, i] = pi
                    if u[b, h, i] < pi:
                        keep[b, h, i] = True
                        w[b, h, i] = np.float32(1.0 / pi)
            idx = np.nonzero(keep[b, h])[0]
            kept_idx[b, h, :idx.size] = idx
            kept_count[b, h] = idx.size
    return dict(tau=tau, p=p, u=u, keep=keep, w=w, kept_idx=kept_idx, kept_count=kept_count)
