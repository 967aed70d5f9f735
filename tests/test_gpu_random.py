"""Randomised GPU parity: forty small problems drawn from a fixed seed, across
the supported space (batch, query and kv heads with every GQA ratio, lengths
with and without a partial last block, d = 64 / 128, block = 64 / 128, causal
or not, bf16 or f32, the budget between 0 and 0.6 or a fixed fraction or top-k,
the softmax scale around 1/sqrt(d)).  Each compares the whole path with the
fp64 oracle to the same bar as the hand-picked cases: kept sets bit-identical,
O, LSE and the gradients within tolerance, skipped dQ rows exactly zero."""
import numpy as np
import pytest

import oracle
from block_sparse_backward_amd import binding as bd
from block_sparse_backward_amd.synth import Config, make_inputs, to_f64
from tests.parity_helpers import LSE_TOL, TOL, host, max_abs_rel, run_gpu

pytestmark = pytest.mark.gpu

RULES = [(bd.SELECT_BUDGET, oracle.RULE_BUDGET), (bd.SELECT_FRACTION, oracle.RULE_FRACTION),
         (bd.SELECT_TOPK, oracle.RULE_TOPK)]


def _draw_cases(n=40, seed=2024):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for c in range(n):
        d = int(rng.choice([64, 128]))
        block = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.choice([1, 2]))
        N = int(rng.integers(1, 9)) * block - int(rng.choice([0, 0, int(rng.integers(1, block))]))
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        causal = bool(rng.random() < 0.7)
        sigma = float(rng.choice([0.5, 1.0, 2.0]))
        rule = int(rng.choice([0, 0, 0, 1, 2]))
        param = float(rng.uniform(0.0, 0.6)) if rule == 0 else float(rng.uniform(0.05, 1.0))
        scale = float(d ** -0.5 * rng.uniform(0.5, 1.5))
        cfg = Config(f"rnd{c}", B, hkv * G, hkv, max(N, 1), d, dtype, causal, block, sigma,
                     boost_frac=0.1 if rng.random() < 0.3 else 0.0, boost=20.0)
        cases.append((cfg, rule, param, scale, int(rng.integers(0, 2**31))))
    return cases


CASES = _draw_cases()


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_random_case_parity(idx):
    cfg, rule, param, scale, seed = CASES[idx]
    print(f"[random] {idx} {cfg} rule={rule} param={param:.4f} scale={scale:.5f} seed={seed}",
          flush=True)
    inp = make_inputs(cfg, seed % 1000)
    dev = "cuda:0"
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
    kw = dict(block=cfg.block, causal=cfg.causal, scale=scale)
    o, lse = bd.attn_fwd(q, k, v, **kw)
    sel = bd.block_select(o, do, param, seed, heads_kv=cfg.Hkv, rule=RULES[rule][0], **kw)
    dq, dk, dv = bd.attn_bwd(q, k, v, lse, do, sel, **kw)

    q64, k64, v64, d64 = (to_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    m_ref = oracle.block_masses(d64, cfg.block)
    ref = oracle.select_rule(m_ref, RULES[rule][1], param, seed)
    assert np.array_equal(host(sel["mass"]), m_ref)
    assert np.array_equal(host(sel["tau"]), ref["tau"], equal_nan=True)
    assert np.array_equal(host(sel["kept_count"]), ref["kept_count"])
    assert np.array_equal(host(sel["kept_idx"]), ref["kept_idx"])
    assert np.array_equal(sel["block_w"].cpu().numpy().view(np.uint32), ref["w"].view(np.uint32))

    o_ref, lse_ref = oracle.attn_fwd(q64, k64, v64, scale, cfg.causal)
    tol = TOL[cfg.dtype]
    assert max_abs_rel(host(o), o_ref) <= tol
    assert np.abs(host(lse) - lse_ref).max() <= LSE_TOL[cfg.dtype]
    g_ref = oracle.attn_bwd_sparse(q64, k64, v64, d64, cfg.block, ref["keep"], ref["w"], scale,
                                   cfg.causal)
    errs = [max_abs_rel(host(x), r) for x, r in zip((dq, dk, dv), g_ref)]
    print(f"[random] {idx} kept={ref['keep'].mean():.3f} errs={errs}", flush=True)
    assert max(errs) <= tol, errs
    skipped = np.repeat(~ref["keep"], cfg.block, axis=2)[:, :, :cfg.N]
    assert np.all(host(dq)[skipped] == 0.0)
