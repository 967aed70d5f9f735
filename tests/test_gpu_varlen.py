"""Variable-length batches through the C ABI: every sequence of the packed
batch matches the fp64 oracle run on that sequence alone (forward, kept set
bit-identical with the sequence index in the draw, sparse backward)."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_backward_amd import binding as bd
from block_sparse_backward_amd.synth import Config, make_inputs, to_f64
from tests.parity_helpers import LSE_TOL, TOL, host, max_abs_rel

pytestmark = pytest.mark.gpu

CASES = {
    # lengths include a zero, a single row, ragged tails and a one-block sequence
    "causal_d128_b128": dict(lens=[300, 1000, 0, 128, 777], Hq=4, Hkv=2, d=128, block=128,
                             causal=True, dtype="bf16", sigma=2.0, delta=0.1, rule="budget"),
    "noncausal_d64_b64": dict(lens=[129, 1, 500], Hq=2, Hkv=2, d=64, block=64, causal=False,
                              dtype="bf16", sigma=1.0, delta=0.2, rule="budget"),
    "f32_causal_topk": dict(lens=[70, 200], Hq=2, Hkv=1, d=64, block=64, causal=True,
                            dtype="f32", sigma=1.5, delta=0.5, rule="topk"),
}
RULES = {"budget": (bd.SELECT_BUDGET, oracle.RULE_BUDGET),
         "topk": (bd.SELECT_TOPK, oracle.RULE_TOPK)}


def _pack(parts):
    return torch.cat([p.reshape(-1) for p in parts]).to("cuda:0")


@pytest.mark.parametrize("name", list(CASES))
def test_varlen_matches_per_sequence_oracle(name):
    c = CASES[name]
    print(f"[varlen] {name} {c}", flush=True)
    lens, Hq, Hkv, d, block = c["lens"], c["Hq"], c["Hkv"], c["d"], c["block"]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(int).tolist()
    cb = bd.varlen_block_offsets(cu, block)
    seqs = []
    for b, L in enumerate(lens):
        cfg = Config(f"v{b}", 1, Hq, Hkv, max(L, 1), d, c["dtype"], c["causal"], block, c["sigma"])
        inp = make_inputs(cfg, 100 + b)
        seqs.append({n: t[:, :, :L] for n, t in inp.items()})
    q, k, v, do = (_pack([s[n][0] for s in seqs]) for n in ("q", "k", "v", "dout"))
    scale = d ** -0.5
    o, lse = bd.attn_fwd_varlen(q, k, v, cu, Hq, Hkv, d, causal=c["causal"], scale=scale,
                                block=block)
    rule = RULES[c["rule"]]
    sel = bd.block_select_varlen(o, do, cu, Hq, d, c["delta"], 9, block=block,
                                 causal=c["causal"], scale=scale, heads_kv=Hkv, rule=rule[0])
    dq, dk, dv = bd.attn_bwd_varlen(q, k, v, lse, do, sel, cu, Hq, Hkv, d, block=block,
                                    causal=c["causal"], scale=scale)
    torch.cuda.synchronize()
    tol = TOL[c["dtype"]]
    for b, L in enumerate(lens):
        nqb = cb[b + 1] - cb[b]
        tau = sel["tau"][Hq * b:Hq * (b + 1)].cpu().numpy()
        cnt = sel["kept_count"][Hq * b:Hq * (b + 1)].cpu().numpy()
        if L == 0:
            assert np.all(np.isinf(tau)) and np.all(cnt == 0)
            continue
        q64, k64, v64, d64 = (to_f64(seqs[b][n]) for n in ("q", "k", "v", "dout"))
        o_ref, lse_ref = oracle.attn_fwd(q64, k64, v64, scale, c["causal"])
        t0 = cu[b]
        sl_q = slice(Hq * t0 * d, Hq * (t0 + L) * d)
        sl_k = slice(Hkv * t0 * d, Hkv * (t0 + L) * d)
        o_b = host(o[sl_q]).reshape(1, Hq, L, d)
        lse_b = host(lse[Hq * t0:Hq * (t0 + L)]).reshape(1, Hq, L)
        assert max_abs_rel(o_b, o_ref) <= tol
        assert np.abs(lse_b - lse_ref).max() <= LSE_TOL[c["dtype"]]
        m = oracle.block_masses(d64, block)
        ref = oracle.select_rule(m, rule[1], c["delta"], 9, b0=b)
        blk = slice(Hq * cb[b], Hq * cb[b + 1])
        assert np.array_equal(sel["mass"][blk].cpu().numpy().reshape(1, Hq, nqb), m)
        assert np.array_equal(tau.reshape(1, Hq), ref["tau"], equal_nan=True)
        assert np.array_equal(cnt.reshape(1, Hq), ref["kept_count"])
        assert np.array_equal(sel["kept_idx"][blk].cpu().numpy().reshape(1, Hq, nqb),
                              ref["kept_idx"])
        assert np.array_equal(sel["block_w"][blk].cpu().numpy().reshape(1, Hq, nqb).view(np.uint32),
                              ref["w"].view(np.uint32))
        g = oracle.attn_bwd_sparse(q64, k64, v64, d64, block, ref["keep"], ref["w"], scale,
                                   c["causal"])
        got = (host(dq[sl_q]).reshape(1, Hq, L, d), host(dk[sl_k]).reshape(1, Hkv, L, d),
               host(dv[sl_k]).reshape(1, Hkv, L, d))
        errs = [max_abs_rel(a, r) for a, r in zip(got, g)]
        print(f"[varlen] {name} seq {b} L={L} kept={ref['keep'].mean():.3f} errs={errs}",
              flush=True)
        assert max(errs) <= tol, (b, errs)


def test_varlen_sequences_draw_independently():
    # two identical sequences in one batch get different uniforms (the draw is
    # keyed by the sequence index), so their kept sets differ
    Hq, d, block, L = 2, 128, 128, 4096
    cfg = Config("vd", 1, Hq, Hq, L, d, "bf16", True, block, 0.5)
    inp = make_inputs(cfg, 0)
    do = _pack([inp["dout"][0], inp["dout"][0]])
    o = torch.zeros_like(do)
    sel = bd.block_select_varlen(o, do, [0, L, 2 * L], Hq, d, 0.3, 1, block=block)
    torch.cuda.synchronize()
    nqb = L // block
    w = sel["block_w"].cpu().numpy().reshape(2, Hq, nqb)
    assert np.array_equal(sel["mass"][:Hq * nqb].cpu().numpy(), sel["mass"][Hq * nqb:].cpu().numpy())
    assert not np.array_equal(w[0] != 0, w[1] != 0)
