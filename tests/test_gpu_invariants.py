"""GPU invariants of the path (through the C ABI): determinism, never-loaded
skipped tiles (NaN poisoning), outputs fully written (NaN-filled buffers),
nesting across budgets, degenerate heads, independence of the backward's two
phases, no state shared between calls on concurrent streams."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_backward_amd import binding as bd
from block_sparse_backward_amd.synth import Config, make_inputs, to_f64
from tests.parity_helpers import TOL, host, max_abs_rel, run_gpu

pytestmark = pytest.mark.gpu

CFG = Config("inv", 1, 8, 2, 1024, 128, "bf16", True, 128, 2.0, boost_frac=0.125, boost=20.0)
CFG64 = Config("inv64", 2, 4, 4, 640, 64, "bf16", False, 64, 1.5)
CFGR = Config("inv_ragged", 1, 8, 2, 1000, 128, "bf16", True, 128, 2.0, boost_frac=0.125,
              boost=20.0)
CFGB64 = Config("inv_d128_b64", 1, 4, 2, 704, 128, "bf16", True, 64, 2.0, boost_frac=0.125,
                boost=20.0)


def _bits(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy() if t.dtype != torch.bool \
        else t.cpu().numpy()


@pytest.mark.parametrize("cfg", [CFG, CFG64], ids=["causal_d128", "noncausal_d64"])
def test_select_and_bwd_are_bit_repeatable(cfg):
    inp = make_inputs(cfg, 0)
    a = run_gpu(cfg, inp, 0.1, seed=3)
    b = run_gpu(cfg, inp, 0.1, seed=3)
    for name in ("mass", "tau", "D", "block_w", "kept_idx", "kept_count"):
        assert np.array_equal(_bits(a["sel"][name]), _bits(b["sel"][name])), name
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(_bits(a[name]), _bits(b[name])), name


@pytest.mark.parametrize("cfg", [CFG, CFG64], ids=["causal_d128", "noncausal_d64"])
def test_skipped_blocks_are_never_read(cfg):
    # Poison Q, dO, LSE and D of every skipped block with NaN after selection:
    # if any kernel of the backward touched them, NaN would spread.
    inp = make_inputs(cfg, 0)
    g = run_gpu(cfg, inp, 0.2, seed=1)
    keep = g["sel"]["block_w"] != 0
    assert 0 < int(keep.sum()) < keep.numel()
    rows = keep.repeat_interleave(cfg.block, dim=2)          # [B, Hq, N]
    qp, dop = g["q"].clone(), g["dout"].clone()
    qp[~rows] = float("nan")
    dop[~rows] = float("nan")
    lsep, sel = g["lse"].clone(), dict(g["sel"])
    lsep[~rows] = float("nan")
    sel["D"] = sel["D"].clone()
    sel["D"][~rows] = float("nan")
    dq, dk, dv = bd.attn_bwd(qp, g["k"], g["v"], lsep, dop, sel, block=cfg.block,
                             causal=cfg.causal, scale=cfg.scale)
    torch.cuda.synchronize()
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.array_equal(_bits(x), _bits(g[name])), name


@pytest.mark.parametrize("cfg", [CFG, CFG64, CFGR, CFGB64],
                         ids=["causal_d128", "noncausal_d64", "ragged", "d128_b64"])
@pytest.mark.parametrize("apart", [False, True], ids=["one_call", "phases_apart"])
def test_outputs_fully_written(cfg, apart):
    # dQ, dK, dV start as NaN: every element must be written, the rows of
    # skipped blocks as exact zeros, whichever kernel writes them (the dK/dV
    # walk in one call, the dQ walk when the phases run apart)
    inp = make_inputs(cfg, 0)
    g = run_gpu(cfg, inp, 0.2, seed=1)
    keep = g["sel"]["block_w"] != 0
    assert 0 < int(keep.sum()) < keep.numel()
    outs = tuple(torch.full_like(g[n], float("nan")) for n in ("dq", "dk", "dv"))
    kw = dict(block=cfg.block, causal=cfg.causal, scale=cfg.scale, out=outs)
    args = (g["q"], g["k"], g["v"], g["lse"], g["dout"], g["sel"])
    if apart:
        bd.attn_bwd(*args, phases=bd.BWD_DQ, **kw)
        bd.attn_bwd(*args, phases=bd.BWD_DKDV, **kw)
    else:
        bd.attn_bwd(*args, **kw)
    torch.cuda.synchronize()
    for name, x in zip(("dq", "dk", "dv"), outs):
        assert not torch.isnan(x).any(), name
        assert np.array_equal(_bits(x), _bits(g[name])), name
    rows = keep.repeat_interleave(cfg.block, dim=2)[:, :, :cfg.N]
    assert int((outs[0][~rows] != 0).sum()) == 0


def test_kept_sets_nest_across_budgets():
    inp = make_inputs(CFG, 0)
    dev = torch.device("cuda:0")
    o = torch.zeros_like(inp["dout"]).to(dev)
    do = inp["dout"].to(dev)
    prev = None
    for dl in (0.0, 0.02, 0.1, 0.3, 0.6, 0.9):
        sel = bd.block_select(o, do, dl, 11, block=CFG.block, causal=CFG.causal,
                              heads_kv=CFG.Hkv)
        keep = (sel["block_w"] != 0).cpu().numpy()
        if prev is not None:
            assert np.all(prev | ~keep)
        prev = keep


def test_nonfinite_and_zero_heads():
    cfg = CFG
    inp = make_inputs(cfg, 0)
    d = inp["dout"].clone()
    d[0, 1, 300, 5] = float("inf")     # head 1: dense fallback, tau NaN
    d[0, 2] = 0.0                      # head 2: all-zero gradient, nothing kept
    inp2 = dict(inp, dout=d)
    g = run_gpu(cfg, inp2, 0.1, seed=2)
    tau = g["sel"]["tau"].cpu().numpy()
    assert math.isnan(tau[0, 1]) and tau[0, 2] == math.inf
    w = g["sel"]["block_w"].cpu().numpy()
    assert np.all(w[0, 1] == 1.0) and g["sel"]["kept_count"][0, 1].item() == cfg.nqb
    assert np.all(w[0, 2] == 0.0) and g["sel"]["kept_count"][0, 2].item() == 0
    assert torch.all(g["dq"][0, 2] == 0)
    # the other heads select exactly as the oracle says
    ref = oracle.select(oracle.block_masses(to_f64(d), cfg.block), 0.1, 2)
    assert np.array_equal(g["sel"]["kept_idx"].cpu().numpy(), ref["kept_idx"])
    # head 1's gradient carries the non-finite value, as the dense backward would
    assert not torch.isfinite(g["dq"][0, 1]).all()


@pytest.mark.parametrize("cfg", [CFG64, CFG, CFGB64], ids=["noncausal_d64", "causal_d128",
                                                          "d128_b64"])
def test_phases_are_independent(cfg):
    # the one call (where d = 128 runs the dQ plan inside the dK/dV launch)
    # and the two phases in reverse order give the same bits
    inp = make_inputs(cfg, 0)
    g = run_gpu(cfg, inp, 0.1, seed=5)
    dq = torch.full_like(g["dq"], 7.0)
    dk = torch.full_like(g["dk"], 7.0)
    dv = torch.full_like(g["dv"], 7.0)
    kw = dict(block=cfg.block, causal=cfg.causal, scale=cfg.scale, out=(dq, dk, dv))
    bd.attn_bwd(g["q"], g["k"], g["v"], g["lse"], g["dout"], g["sel"], phases=bd.BWD_DQ, **kw)
    torch.cuda.synchronize()
    assert torch.all(dk == 7.0) and torch.all(dv == 7.0)
    bd.attn_bwd(g["q"], g["k"], g["v"], g["lse"], g["dout"], g["sel"], phases=bd.BWD_DKDV, **kw)
    torch.cuda.synchronize()
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.array_equal(_bits(x), _bits(g[name])), name


def test_empty_problem_is_a_noop():
    dev = torch.device("cuda:0")
    q = torch.empty((0, 4, 256, 64), dtype=torch.bfloat16, device=dev)
    k = torch.empty((0, 2, 256, 64), dtype=torch.bfloat16, device=dev)
    o, lse = bd.attn_fwd(q, k, k, causal=True, block=64)
    sel = bd.block_select(o, q, 0.1, 0, block=64, heads_kv=2)
    dq, dk, dv = bd.attn_bwd(q, k, k, lse, q, sel, block=64)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and dk.numel() == 0


def test_delta_zero_is_the_dense_gradient():
    cfg = CFG64
    inp = make_inputs(cfg, 0)
    g = run_gpu(cfg, inp, 0.0, seed=0)
    assert torch.all(g["sel"]["block_w"] == 1.0)
    q64, k64, v64, d64 = (to_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    ref = oracle.attn_bwd_dense(q64, k64, v64, d64, cfg.scale, cfg.causal)
    for name, r in zip(("dq", "dk", "dv"), ref):
        assert max_abs_rel(host(g[name]), r) <= TOL["bf16"], name


def test_concurrent_streams_share_no_state():
    """Two problems of different shapes run at the same time on two streams
    (each with its own outputs and workspace) give the bits of the same problems
    run one after the other: the library keeps no state between calls."""
    dev = torch.device("cuda:0")
    cfgs = [(CFG, 0.1, 3), (CFGB64, 0.2, 4)]

    def setup(cfg, delta, seed):
        inp = make_inputs(cfg, seed)
        q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
        o, lse = torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        sel = bd.select_outputs(cfg.B, cfg.Hq, cfg.N, cfg.block, dev)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        ws = bd.bwd_workspace(q, k, cfg.block, cfg.causal)
        kw = dict(block=cfg.block, causal=cfg.causal, scale=cfg.scale)

        def run():
            for _ in range(3):  # repeated, so that the two streams overlap for a while
                bd.attn_fwd(q, k, v, out=(o, lse), **kw)
                bd.block_select(o, do, delta, seed, heads_kv=cfg.Hkv, out=sel, **kw)
                bd.attn_bwd(q, k, v, lse, do, sel, out=grads, workspace=ws, **kw)

        def outs():
            return [_bits(t) for t in (o, lse, *grads, sel["kept_idx"], sel["block_w"])]
        return run, outs

    jobs = [setup(*c) for c in cfgs]
    ref = []
    for run, outs in jobs:
        run()
        torch.cuda.synchronize()
        ref.append(outs())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for (run, _), s in zip(jobs, streams):
        with torch.cuda.stream(s):
            run()
    torch.cuda.synchronize()
    for (_, outs), r in zip(jobs, ref):
        for a, b in zip(outs(), r):
            assert np.array_equal(a, b)


def test_misaligned_tensor_refused_before_any_launch():
    # a contiguous view two bytes into its storage: the library moves element
    # tensors in 16-byte pieces, so it refuses the pointer and launches nothing
    dev = torch.device("cuda:0")
    B, Hq, Hkv, N, d = 1, 2, 1, 256, 64
    n = B * Hq * N * d
    base = torch.zeros(n + 8, dtype=torch.bfloat16, device=dev)
    q_mis = base[1:1 + n].view(B, Hq, N, d)
    assert q_mis.is_contiguous() and q_mis.data_ptr() % 16 == 2
    k = torch.zeros((B, Hkv, N, d), dtype=torch.bfloat16, device=dev)
    with pytest.raises(bd.LazyFlashError, match="misaligned"):
        bd.attn_fwd(q_mis, k, k, causal=True, block=64)
    o, lse = bd.attn_fwd(q_mis.clone(), k, k, causal=True, block=64)  # aligned copy runs
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
