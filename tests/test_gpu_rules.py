"""GPU parity of the other selection rules (fixed fraction, top-k) through the
C ABI: kept sets, tau and weights bit-identical to the fp64 oracle, and the
unchanged backward over each rule's selection within tolerance.  These are the
rules the budget is compared with at equal backward time (LazyFlash entry on
gyom.fr, section "Le choix des blocs pèse plus que la quantité sautée")."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_backward_amd import binding as bd
from block_sparse_backward_amd.synth import Config, make_inputs, to_f64
from tests.parity_helpers import TOL, host, max_abs_rel

pytestmark = pytest.mark.gpu

RULES = {"fraction": (bd.SELECT_FRACTION, oracle.RULE_FRACTION),
         "topk": (bd.SELECT_TOPK, oracle.RULE_TOPK)}


def _select(cfg, o, do, rule, f, seed):
    sel = bd.block_select(o, do, f, seed, block=cfg.block, causal=cfg.causal, scale=cfg.scale,
                          heads_kv=cfg.Hkv, rule=RULES[rule][0])
    torch.cuda.synchronize()
    return sel


def _check_exact(sel, ref, mass_ref):
    assert np.array_equal(sel["mass"].cpu().numpy(), mass_ref, equal_nan=True)
    assert np.array_equal(sel["tau"].cpu().numpy(), ref["tau"], equal_nan=True)
    assert np.array_equal(sel["kept_count"].cpu().numpy(), ref["kept_count"])
    assert np.array_equal(sel["kept_idx"].cpu().numpy(), ref["kept_idx"])
    assert np.array_equal(sel["block_w"].cpu().numpy().view(np.uint32), ref["w"].view(np.uint32))


CFG = Config("rules", 2, 8, 2, 2048, 128, "bf16", True, 128, 2.0, boost_frac=0.1, boost=20.0)
CFG64 = Config("rules64", 1, 4, 4, 4096, 64, "bf16", False, 64, 1.0)


@pytest.mark.parametrize("rule", list(RULES))
@pytest.mark.parametrize("f", [0.04, 0.3, 0.77, 1.0])
@pytest.mark.parametrize("cfg", [CFG, CFG64], ids=["gqa_d128_b128", "mha_d64_b64"])
def test_rule_selection_bit_exact(cfg, rule, f):
    print(f"[rules] {cfg.name} {rule} f={f}", flush=True)
    inp = make_inputs(cfg, 0)
    q, k, v, do = (inp[n].to("cuda:0") for n in ("q", "k", "v", "dout"))
    o, _ = bd.attn_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale, block=cfg.block)
    m = oracle.block_masses(to_f64(inp["dout"]), cfg.block)
    for seed in (0, 11):
        sel = _select(cfg, o, do, rule, f, seed)
        _check_exact(sel, oracle.select_rule(m, RULES[rule][1], f, seed), m)


def test_rules_with_ties_zero_blocks_and_a_nonfinite_head():
    # dO constant over blocks 0..7 (equal masses: top-k ties), zero over blocks
    # 8..11 (never kept), a NaN in head 2 (dense fallback).
    cfg = Config("ties", 1, 3, 1, 16 * 64, 64, "bf16", True, 64, 1.0)
    inp = make_inputs(cfg, 0)
    do = inp["dout"].clone()
    do[:, :, :8 * 64] = 0.5
    do[:, :, 8 * 64:12 * 64] = 0.0
    do[0, 2, 100, 3] = float("nan")
    o = torch.zeros_like(do)
    m = oracle.block_masses(to_f64(do), cfg.block)
    dd, oo = do.to("cuda:0"), o.to("cuda:0")
    for rule in RULES:
        for f in (0.1, 0.5, 0.9, 1.0):
            sel = _select(cfg, oo, dd, rule, f, 5)
            ref = oracle.select_rule(m, RULES[rule][1], f, 5)
            _check_exact(sel, ref, m)
    ref = oracle.select_rule(m, oracle.RULE_TOPK, 0.5, 5)
    # 12 positive blocks per head, k = 6: the 4 larger random blocks, then the
    # lowest-index two of the 8 tied constant blocks
    assert ref["kept_count"][0, 0] == 6 and ref["keep"][0, 0, :2].all()
    assert not ref["keep"][0, 0, 2:12].any()


def test_rules_at_the_largest_block_count():
    cfg = Config("maxnqb", 1, 2, 1, 4096 * 64, 64, "bf16", True, 64, 2.0, boost_frac=0.05, boost=20.0)
    inp = make_inputs(cfg, 0)
    do = inp["dout"].to("cuda:0")
    o = torch.zeros_like(do)
    m = oracle.block_masses(to_f64(inp["dout"]), cfg.block)
    for rule, f in (("fraction", 0.05), ("topk", 0.05), ("fraction", 0.6), ("topk", 0.6)):
        sel = _select(cfg, o, do, rule, f, 3)
        _check_exact(sel, oracle.select_rule(m, RULES[rule][1], f, 3), m)


@pytest.mark.parametrize("rule", list(RULES))
def test_backward_over_rule_selection(rule):
    cfg = Config("rulesbwd", 1, 4, 2, 768, 128, "bf16", True, 128, 2.0, boost_frac=0.2, boost=20.0)
    inp = make_inputs(cfg, 0)
    q, k, v, do = (inp[n].to("cuda:0") for n in ("q", "k", "v", "dout"))
    o, lse = bd.attn_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale, block=cfg.block)
    sel = _select(cfg, o, do, rule, 0.35, 2)
    dq, dk, dv = bd.attn_bwd(q, k, v, lse, do, sel, block=cfg.block, causal=cfg.causal,
                             scale=cfg.scale)
    torch.cuda.synchronize()
    q64, k64, v64, d64 = (to_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    ref = oracle.select_rule(oracle.block_masses(d64, cfg.block), RULES[rule][1], 0.35, 2)
    g = oracle.attn_bwd_sparse(q64, k64, v64, d64, cfg.block, ref["keep"], ref["w"], cfg.scale,
                               cfg.causal)
    errs = [max_abs_rel(host(x), r) for x, r in zip((dq, dk, dv), g)]
    print(f"[rules] bwd {rule} kept={ref['keep'].mean():.3f} errs={errs}", flush=True)
    assert max(errs) <= TOL["bf16"], errs
