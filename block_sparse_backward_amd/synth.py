"""Seeded synthetic inputs (Q, K, V, dO) shared by the tests, the benchmark and
the oracle checks.

This module holds no part of the attention or selection arithmetic: it only
draws random tensors of the workload's shape and value distribution.

Recipe (the LazyFlash journal entry measures on LongAlign examples with a
Qwen3-8B model; neither data nor weights are used here, synthetic tensors of
the same layer shape stand in for them):

* generator: numpy ``Generator(PCG64(data_seed))``, draws in this order:
  Q, K, V, the dO base, the per-row log-scales, the boosted blocks;
* Q, K, V ~ N(0, 1), float32;
* dO = N(0, 1) * exp(sigma * Z), Z ~ N(0, 1) independent per (b, h, row), so
  each row is scaled by a lognormal(0, sigma) factor;
* optionally ``boost_frac`` of the query blocks of every (b, h), chosen
  uniformly without replacement, have their dO rows multiplied by ``boost``;
* all tensors are generated in float32 and rounded once (round-to-nearest-
  even, torch CPU cast) to the storage dtype; the very same bits go to the GPU
  and, upcast to float64, to the oracle.
"""
from dataclasses import dataclass, field, replace

import numpy as np
import torch

__all__ = ["Config", "CONFIGS", "make_inputs", "to_f64"]


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str          # "bf16" or "f32"
    causal: bool
    block: int
    sigma: float        # std of the log of the per-row dO scale
    deltas: tuple = field(default=(0.1,))
    boost_frac: float = 0.0
    boost: float = 1.0

    @property
    def nqb(self):
        return -(-self.N // self.block)  # the last block may be partial

    @property
    def scale(self):
        return 1.0 / float(np.sqrt(self.d))

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    "tiny": Config("tiny", 1, 2, 2, 256, 64, "f32", True, 64, 1.0, (0.1,)),
    "mid": Config("mid", 1, 32, 8, 8192, 128, "bf16", True, 128, 1.5, (0.0, 0.05, 0.1)),
    "headline": Config("headline", 1, 32, 8, 32768, 128, "bf16", True, 128, 2.0,
                       (0.0, 0.1, 0.2), boost_frac=0.05, boost=20.0),
    "long": Config("long", 1, 32, 8, 65536, 128, "bf16", True, 128, 2.0, (0.1,)),
    "noncausal": Config("noncausal", 4, 16, 16, 16384, 64, "bf16", False, 64, 0.25, (0.02, 0.1)),
}


def make_inputs(cfg: Config, data_seed: int = 0):
    """Return dict(q, k, v, dout) of CPU torch tensors in ``cfg.torch_dtype``.

    q, dout: [B, Hq, N, d]; k, v: [B, Hkv, N, d]; row-major, d fastest.
    """
    rng = np.random.Generator(np.random.PCG64(data_seed))
    qs = (cfg.B, cfg.Hq, cfg.N, cfg.d)
    ks = (cfg.B, cfg.Hkv, cfg.N, cfg.d)
    q = rng.standard_normal(qs, dtype=np.float32)
    k = rng.standard_normal(ks, dtype=np.float32)
    v = rng.standard_normal(ks, dtype=np.float32)
    do = rng.standard_normal(qs, dtype=np.float32)
    z = rng.standard_normal((cfg.B, cfg.Hq, cfg.N), dtype=np.float32)
    do *= np.exp(np.float32(cfg.sigma) * z)[..., None]
    nboost = int(round(cfg.boost_frac * cfg.nqb))
    if nboost:
        for b in range(cfg.B):
            for h in range(cfg.Hq):
                blocks = rng.choice(cfg.nqb, size=nboost, replace=False)
                for i in blocks:
                    do[b, h, i * cfg.block:(i + 1) * cfg.block] *= np.float32(cfg.boost)
    td = cfg.torch_dtype
    return {name: torch.from_numpy(a).to(td)
            for name, a in (("q", q), ("k", k), ("v", v), ("dout", do))}


def to_f64(t):
    """Exact float64 numpy copy of a CPU torch tensor (bf16 or f32)."""
    return t.to(torch.float64).numpy()
