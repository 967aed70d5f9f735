"""The training-time wrapper (torch.autograd.Function over the C ABI) against
the fp64 oracle: gradients of o.backward(dO) equal the oracle's sparse
gradient for the oracle's own kept set, the dense gradient at delta = 0, and a
new seed per step redraws the selection."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_backward_amd.autograd import draw_seed, lazyflash_attention
from block_sparse_backward_amd.synth import Config, make_inputs, to_f64
from tests.parity_helpers import LSE_TOL, TOL, host, max_abs_rel

pytestmark = pytest.mark.gpu

CASES = {
    "gqa_causal_d128_b128": (Config("ag1", 1, 4, 2, 512, 128, "bf16", True, 128, 2.0,
                                    boost_frac=0.125, boost=20.0), 0.1),
    "gqa_causal_d64_b64_dense": (Config("ag2", 2, 4, 1, 448, 64, "bf16", True, 64, 1.5), 0.0),
    "noncausal_d64_b64": (Config("ag3", 1, 2, 2, 384, 64, "bf16", False, 64, 1.0), 0.2),
    "f32_causal_d64": (Config("ag4", 1, 2, 1, 256, 64, "f32", True, 64, 1.0), 0.1),
}


def _leaf(t):
    return t.to("cuda:0").requires_grad_(True)


@pytest.mark.parametrize("name", list(CASES))
def test_autograd_gradients_match_oracle(name):
    cfg, delta = CASES[name]
    print(f"[autograd] {name} {cfg} delta={delta}", flush=True)
    inp = make_inputs(cfg, 0)
    seed = draw_seed(step=7, layer=3)
    q, k, v = (_leaf(inp[n]) for n in ("q", "k", "v"))
    stats = {}
    o = lazyflash_attention(q, k, v, delta, seed, causal=cfg.causal, scale=cfg.scale,
                            block=cfg.block, stats=stats)
    o.backward(inp["dout"].to("cuda:0"))
    torch.cuda.synchronize()

    q64, k64, v64, d64 = (to_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    o_ref, _ = oracle.attn_fwd(q64, k64, v64, cfg.scale, cfg.causal)
    ref = oracle.select(oracle.block_masses(d64, cfg.block), delta, seed)
    assert np.array_equal(stats["kept_count"].cpu().numpy(), ref["kept_count"])
    assert np.array_equal(stats["block_w"].cpu().numpy().view(np.uint32),
                          ref["w"].view(np.uint32))
    tol = TOL[cfg.dtype]
    assert max_abs_rel(host(o), o_ref) <= tol
    dq, dk, dv = oracle.attn_bwd_sparse(q64, k64, v64, d64, cfg.block, ref["keep"], ref["w"],
                                        cfg.scale, cfg.causal)
    errs = [max_abs_rel(host(t.grad), r) for t, r in ((q, dq), (k, dk), (v, dv))]
    print(f"[autograd] {name} kept={ref['keep'].mean():.3f} errs={errs}", flush=True)
    assert max(errs) <= tol, errs
    if delta == 0.0:
        dense = oracle.attn_bwd_dense(q64, k64, v64, d64, cfg.scale, cfg.causal)
        for t, r in zip((q, k, v), dense):
            assert max_abs_rel(host(t.grad), r) <= tol


def test_autograd_accepts_views_and_accumulates_into_leaves():
    # Non-contiguous inputs (a transposed [B, N, H, d] layout) and a loss that
    # is not o itself: the gradient reaching o is 2*o*dO' computed by torch,
    # the wrapper must take it as dO.
    cfg = Config("ag5", 1, 4, 2, 256, 64, "bf16", True, 64, 1.0)
    inp = make_inputs(cfg, 0)
    qt, kt, vt = (inp[n].transpose(1, 2).contiguous().to("cuda:0").requires_grad_(True)
                  for n in ("q", "k", "v"))
    q, k, v = (t.transpose(1, 2) for t in (qt, kt, vt))
    assert not q.is_contiguous()
    o = lazyflash_attention(q, k, v, 0.0, 0, causal=True, scale=cfg.scale, block=cfg.block)
    w = inp["dout"].to("cuda:0")
    (o.float() * w.float()).sum().backward()
    torch.cuda.synchronize()
    q64, k64, v64, w64 = (to_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    dq, dk, dv = oracle.attn_bwd_dense(q64, k64, v64, w64, cfg.scale, True)
    for t, r in ((qt, dq), (kt, dk), (vt, dv)):
        assert max_abs_rel(host(t.grad.transpose(1, 2)), r) <= TOL["bf16"]


def test_autograd_accepts_misaligned_contiguous_inputs():
    # contiguous views two bytes into their storage: the library refuses such
    # pointers, so the wrapper copies them; the result is the aligned one's
    cfg = Config("ag7", 1, 4, 2, 256, 64, "bf16", True, 64, 1.0)
    inp = make_inputs(cfg, 0)
    dev = torch.device("cuda:0")

    def offset_copy(t):
        base = torch.zeros(t.numel() + 8, dtype=t.dtype, device=dev)
        view = base[1:1 + t.numel()].view(t.shape)
        view.copy_(t.to(dev))
        assert view.is_contiguous() and view.data_ptr() % 16 != 0
        return view

    grads = []
    for make in (lambda t: t.to(dev).clone(), offset_copy):
        leaves = [make(inp[n]).requires_grad_(True) for n in ("q", "k", "v")]
        o = lazyflash_attention(*leaves, 0.1, 3, causal=True, scale=cfg.scale, block=cfg.block)
        o.backward(offset_copy(inp["dout"]) if make is offset_copy else inp["dout"].to(dev))
        torch.cuda.synchronize()
        grads.append([o.detach()] + [t.grad for t in leaves])
    for a, b in zip(*grads):
        assert torch.equal(a, b)


def test_new_seed_redraws_and_same_seed_repeats():
    cfg = Config("ag6", 1, 4, 2, 1024, 128, "bf16", True, 128, 1.0)
    inp = make_inputs(cfg, 0)
    q, k, v = (inp[n].to("cuda:0") for n in ("q", "k", "v"))
    do = inp["dout"].to("cuda:0")

    def grads(seed):
        qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
        st = {}
        lazyflash_attention(qq, kk, vv, 0.3, seed, block=cfg.block, stats=st).backward(do)
        torch.cuda.synchronize()
        return [t.grad.clone() for t in (qq, kk, vv)], st["block_w"].clone()

    (g1, w1), (g2, w2), (g3, w3) = grads(draw_seed(0)), grads(draw_seed(0)), grads(draw_seed(1))
    assert all(torch.equal(a, b) for a, b in zip(g1, g2)) and torch.equal(w1, w2)
    assert not torch.equal(w1 != 0, w3 != 0)
    m = oracle.block_masses(to_f64(inp["dout"]), cfg.block)
    for s, w in ((draw_seed(0), w1), (draw_seed(1), w3)):
        assert np.array_equal(w.cpu().numpy().view(np.uint32),
                              oracle.select(m, 0.3, s)["w"].view(np.uint32))


@pytest.mark.parametrize("rule", ["fraction", "topk"])
def test_autograd_with_other_selection_rules(rule):
    from block_sparse_backward_amd import binding as bd
    codes = {"fraction": (bd.SELECT_FRACTION, oracle.RULE_FRACTION),
             "topk": (bd.SELECT_TOPK, oracle.RULE_TOPK)}[rule]
    cfg = Config("ag7", 1, 4, 2, 512, 128, "bf16", True, 128, 2.0, boost_frac=0.25, boost=20.0)
    inp = make_inputs(cfg, 0)
    q, k, v = (_leaf(inp[n]) for n in ("q", "k", "v"))
    stats = {}
    o = lazyflash_attention(q, k, v, 0.4, 13, scale=cfg.scale, block=cfg.block, stats=stats,
                            rule=codes[0])
    o.backward(inp["dout"].to("cuda:0"))
    torch.cuda.synchronize()
    q64, k64, v64, d64 = (to_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    ref = oracle.select_rule(oracle.block_masses(d64, cfg.block), codes[1], 0.4, 13)
    assert np.array_equal(stats["block_w"].cpu().numpy().view(np.uint32), ref["w"].view(np.uint32))
    g = oracle.attn_bwd_sparse(q64, k64, v64, d64, cfg.block, ref["keep"], ref["w"], cfg.scale,
                               True)
    errs = [max_abs_rel(host(t.grad), r) for t, r in zip((q, k, v), g)]
    assert max(errs) <= TOL["bf16"], errs
