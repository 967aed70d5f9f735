"""Attention as used in training: a dense forward and a backward over the
query blocks that the gradient-mass budget keeps.

The LazyFlash journal entry on gyom.fr ("LazyFlash allège la
rétropropagation de l'attention, 5,72 fois") describes this use:
  - the forward is ordinary exact attention and saves O and the logsumexp
    (section "Le passage arrière fait deux fois le travail du passage avant");
  - at each backward step, per head, query blocks are ranked by the mass of
    their output gradient and drawn under the budget delta, with a fresh draw
    at every step (section "Un budget sur la masse de gradient, et un tirage
    qui garde le gradient non biaisé");
  - the backward kernel consumes the per-block weights (section "Trois
    tailles de modèle, 19 découpages sur 21").

`LazyFlashAttention` is a torch.autograd.Function around the three C-ABI
calls; every step of the computation runs in the HIP library.  The seed of
the draw must change from one step (and layer) to the next: `draw_seed` packs
(base, step, layer) into a distinct 64-bit seed.
"""
import torch

from . import binding

__all__ = ["LazyFlashAttention", "lazyflash_attention", "draw_seed"]

_STEP_BITS, _LAYER_BITS = 32, 16


def draw_seed(step, layer=0, base=0):
    """A distinct 64-bit seed per (base, step, layer): base in [0, 2^16),
    step in [0, 2^32), layer in [0, 2^16).  The Philox draw keyed by it is
    then independent across steps and layers."""
    if not (0 <= base < 1 << 16 and 0 <= step < 1 << _STEP_BITS and 0 <= layer < 1 << _LAYER_BITS):
        raise ValueError(f"draw_seed: base {base}, step {step} or layer {layer} out of range")
    return (base << (_STEP_BITS + _LAYER_BITS)) | (step << _LAYER_BITS) | layer


def _dense(t):
    """t contiguous and on a 16-byte boundary (the library moves element
    tensors in 16-byte pieces and refuses other pointers): a copy only when
    t is neither."""
    t = t.contiguous()
    return t if t.data_ptr() % 16 == 0 else t.clone()


class LazyFlashAttention(torch.autograd.Function):
    """o = attention(q, k, v); backward = block selection + sparse backward.

    q [B, Hq, N, d], k and v [B, Hkv, N, d]: GPU tensors, bfloat16 or float32
    (copied here when not contiguous or not on a 16-byte boundary).  delta in [0, 1) is the budget on the discarded
    gradient mass (0 keeps every block: the exact dense gradient); seed keys
    the draw.  If `stats` is a dict, the backward stores in it the selection's
    device tensors (mass, tau, block_w, kept_idx, kept_count) without waiting
    for them.  `rule` (binding.SELECT_*) swaps the budget for a fixed-fraction
    or top-k selection, delta then being the kept fraction."""

    @staticmethod
    def forward(ctx, q, k, v, delta, seed, causal, scale, block, stats, rule=binding.SELECT_BUDGET):
        q, k, v = _dense(q), _dense(k), _dense(v)
        o, lse = binding.attn_fwd(q, k, v, causal=causal, scale=scale, block=block)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.cfg = (float(delta), int(seed), bool(causal), scale, int(block), stats, int(rule))
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        delta, seed, causal, scale, block, stats, rule = ctx.cfg
        do = _dense(do.to(q.dtype))
        sel = binding.block_select(o, do, delta, seed, block=block, causal=causal, scale=scale,
                                   heads_kv=k.shape[1], rule=rule)
        dq, dk, dv = binding.attn_bwd(q, k, v, lse, do, sel, block=block, causal=causal,
                                      scale=scale)
        if stats is not None:
            stats.update({n: sel[n] for n in ("mass", "tau", "block_w", "kept_idx",
                                              "kept_count")})
        return dq, dk, dv, None, None, None, None, None, None, None


def lazyflash_attention(q, k, v, delta, seed, causal=True, scale=None, block=128, stats=None,
                        rule=binding.SELECT_BUDGET):
    """Functional form of LazyFlashAttention (scale defaults to 1/sqrt(d)).
    `rule` selects the blocks by the budget (default; `delta` is the budget)
    or, for comparisons, by a fixed fraction or top-k (`delta` is then the
    kept fraction in (0, 1])."""
    d = float(delta)
    if rule == binding.SELECT_BUDGET:
        if not 0.0 <= d < 1.0:
            raise ValueError(f"delta must lie in [0, 1), got {delta}")
    elif rule in (binding.SELECT_FRACTION, binding.SELECT_TOPK):
        if not 0.0 < d <= 1.0:
            raise ValueError(f"the kept fraction must lie in (0, 1], got {delta}")
    else:
        raise ValueError(f"unknown selection rule {rule}")
    return LazyFlashAttention.apply(q, k, v, delta, seed, causal, scale, block, stats, rule)
