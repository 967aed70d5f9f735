"""The whole path (forward, selection, sparse backward) captured once in a HIP
graph and replayed: the library launches kernels only (no allocation, no host
synchronisation, no memset), so every replay must reproduce the eager run's
outputs bit for bit, also with other eager work on the same buffers between
the replays."""
import pytest
import torch

from block_sparse_backward_amd import binding as bd
from block_sparse_backward_amd.synth import Config, make_inputs

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_causal_gqa_d128_b128": (Config("g1", 1, 8, 2, 1024, 128, "bf16", True, 128, 2.0,
                                         boost_frac=0.1, boost=20.0), 0.1),
    "bf16_noncausal_d64_b64_ragged": (Config("g2", 2, 4, 4, 700, 64, "bf16", False, 64, 1.0), 0.2),
    "bf16_dense_delta0": (Config("g3", 1, 4, 1, 512, 128, "bf16", True, 64, 1.5), 0.0),
}


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _snapshot(o, lse, sel, grads):
    out = {"o": o, "lse": lse, "dq": grads[0], "dk": grads[1], "dv": grads[2]}
    out.update({f"sel.{n}": t for n, t in sel.items()})
    return {n: _bits(t).clone() for n, t in out.items()}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    cfg, delta = CASES[name]
    print(f"[graph] {name} {cfg} delta={delta}", flush=True)
    inp = make_inputs(cfg, 0)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
    kw = dict(block=cfg.block, causal=cfg.causal, scale=cfg.scale)
    o, lse = torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    sel = bd.select_outputs(cfg.B, cfg.Hq, cfg.N, cfg.block, dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ws = bd.bwd_workspace(q, k, cfg.block, cfg.causal)

    def step():
        bd.attn_fwd(q, k, v, out=(o, lse), **kw)
        bd.block_select(o, do, delta, 11, heads_kv=cfg.Hkv, out=sel, **kw)
        bd.attn_bwd(q, k, v, lse, do, sel, out=grads, workspace=ws, **kw)

    step()
    torch.cuda.synchronize()
    ref = _snapshot(o, lse, sel, grads)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream's side, as torch recommends
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    other = bd.select_outputs(cfg.B, cfg.Hq, cfg.N, cfg.block, dev)
    for rep in range(3):
        # eager work between replays: scribble over every output, run another draw
        for t in (o, lse, *grads, sel["D"], sel["mass"], sel["tau"], sel["block_w"]):
            t.fill_(float("nan"))
        sel["kept_idx"].fill_(-7)
        sel["kept_count"].fill_(-7)
        bd.block_select(o.clone().fill_(1.0), do, 0.5, 1000 + rep, heads_kv=cfg.Hkv, out=other, **kw)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(o, lse, sel, grads)
        for n in ref:
            assert torch.equal(got[n], ref[n]), f"replay {rep}: {n} differs from the eager run"
    print(f"[graph] {name} 3 replays bit-identical", flush=True)
