"""lf_attn_bwd_noalloc (static device scratch, no allocation) against
lf_attn_bwd (caller workspace) through the C ABI: the same kernels, so the
outputs must be bit-identical.  Calls follow one another on one GPU with
shrinking problems, so each call finds the previous call's contents in the
shared scratch: a 4096-row problem whose few kept blocks the dQ plan cuts into
chunks (fp32 partials in the scratch), then a smaller ragged d = 64 problem,
then an fp32 one (no scratch)."""
import pytest
import torch

from block_sparse_backward_amd import binding as bd
from block_sparse_backward_amd.synth import Config, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    (Config("na1", 1, 8, 2, 4096, 128, "bf16", True, 128, 2.0, boost_frac=0.05, boost=20.0), 0.1),
    (Config("na2", 2, 4, 1, 1000, 64, "bf16", True, 64, 1.5), 0.05),
    (Config("na3", 1, 2, 2, 200, 64, "f32", False, 64, 1.0), 0.1),
]


def _problem(cfg, delta, seed):
    dev = torch.device("cuda:0")
    inp = make_inputs(cfg, 0)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
    o, lse = bd.attn_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale, block=cfg.block)
    sel = bd.block_select(o, do, delta, seed, block=cfg.block, causal=cfg.causal,
                          scale=cfg.scale, heads_kv=cfg.Hkv)
    return q, k, v, lse, do, sel


def test_noalloc_matches_workspace_backward_on_consecutive_calls():
    for round_ in range(2):
        for cfg, delta in CASES:
            print(f"[noalloc] round {round_} {cfg} delta={delta}", flush=True)
            q, k, v, lse, do, sel = _problem(cfg, delta, seed=round_)
            kw = dict(block=cfg.block, causal=cfg.causal, scale=cfg.scale)
            want = bd.attn_bwd(q, k, v, lse, do, sel, **kw)
            # NaN-filled outputs: every element must be written by the call
            out = tuple(torch.full_like(t, float("nan")) for t in want)
            got = bd.attn_bwd_noalloc(q, k, v, lse, do, sel, out=out, **kw)
            torch.cuda.synchronize()
            assert int((sel["block_w"] != 0).sum()) > 0
            for name, g, w in zip(("dq", "dk", "dv"), got, want):
                assert torch.equal(g, w), f"{name} differs in {cfg.name}"


def test_noalloc_backward_replays_in_a_graph():
    # The caller it is for: a backward captured in a HIP graph with every
    # buffer preallocated.  The first call on the GPU (eager, before the
    # capture) looks up the static array's address; the captured call then
    # only launches kernels.  Replays, with the outputs scribbled over and
    # another backward on the same static array run eagerly in between, must
    # give the eager result bit for bit.
    cfg, delta = CASES[0]
    q, k, v, lse, do, sel = _problem(cfg, delta, seed=5)
    kw = dict(block=cfg.block, causal=cfg.causal, scale=cfg.scale)
    out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    bd.attn_bwd_noalloc(q, k, v, lse, do, sel, out=out, **kw)
    torch.cuda.synchronize()
    ref = tuple(t.clone() for t in out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bd.attn_bwd_noalloc(q, k, v, lse, do, sel, out=out, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bd.attn_bwd_noalloc(q, k, v, lse, do, sel, out=out, **kw)
    torch.cuda.synchronize()
    cfg2, delta2 = CASES[1]
    other = _problem(cfg2, delta2, seed=9)
    for rep in range(3):
        for t in out:
            t.fill_(float("nan"))
        bd.attn_bwd_noalloc(*other, block=cfg2.block, causal=cfg2.causal, scale=cfg2.scale)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), out, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
