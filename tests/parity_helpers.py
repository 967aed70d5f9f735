"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same seeded inputs, compare."""
import math

import numpy as np
import torch

import oracle
from block_sparse_backward_amd import binding as bd
from block_sparse_backward_amd.synth import make_inputs, to_f64

TOL = {"bf16": 2e-2, "f32": 1e-4}          # max-abs-rel on O, dQ, dK, dV
LSE_TOL = {"bf16": 1e-3, "f32": 1e-5}      # max-abs on LSE


def max_abs_rel(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    num = np.abs(x - ref).max()
    if den == 0.0:
        return float(num)
    return float(num / den)


def run_gpu(cfg, inp, delta, seed, device="cuda:0", scale=None):
    """fwd -> select -> bwd on the GPU (softmax scale cfg.scale unless given);
    returns (device tensors dict)."""
    scale = cfg.scale if scale is None else scale
    q, k, v, do = (inp[n].to(device) for n in ("q", "k", "v", "dout"))
    o, lse = bd.attn_fwd(q, k, v, causal=cfg.causal, scale=scale, block=cfg.block)
    sel = bd.block_select(o, do, delta, seed, block=cfg.block, causal=cfg.causal,
                          scale=scale, heads_kv=cfg.Hkv)
    dq, dk, dv = bd.attn_bwd(q, k, v, lse, do, sel, block=cfg.block, causal=cfg.causal,
                             scale=scale)
    torch.cuda.synchronize(device)
    return dict(q=q, k=k, v=v, dout=do, o=o, lse=lse, sel=sel, dq=dq, dk=dk, dv=dv)


def host(t):
    return t.detach().to("cpu").to(torch.float64).numpy() if t.is_floating_point() \
        else t.detach().to("cpu").numpy()


def check_select_exact(cfg, inp, gpu, delta, seed):
    """mass, tau, block_w, kept_idx, kept_count bit-identical to the oracle."""
    d64 = to_f64(inp["dout"])
    m_ref = oracle.block_masses(d64, cfg.block)
    ref = oracle.select(m_ref, delta, seed)
    sel = gpu["sel"]
    m_gpu = sel["mass"].cpu().numpy()
    assert np.array_equal(m_gpu, m_ref), "mass differs: %r" % (np.argwhere(m_gpu != m_ref)[:5],)
    tau = sel["tau"].cpu().numpy()
    assert np.array_equal(tau, ref["tau"], equal_nan=True), (tau, ref["tau"])
    assert np.array_equal(sel["kept_count"].cpu().numpy(), ref["kept_count"])
    assert np.array_equal(sel["kept_idx"].cpu().numpy(), ref["kept_idx"])
    w = sel["block_w"].cpu().numpy()
    assert np.array_equal(w.view(np.uint32), ref["w"].view(np.uint32))
    return ref


def check_fwd_rows(cfg, inp, gpu, heads, rows):
    """O and LSE of the given (b, h) heads and query rows vs the oracle."""
    q64, k64, v64 = (to_f64(inp[n]) for n in ("q", "k", "v"))
    G = cfg.Hq // cfg.Hkv
    o_g = gpu["o"]
    lse_g = gpu["lse"]
    errs, lerr = [], 0.0
    o_all, r_all = [], []
    for b, h in heads:
        o_r, l_r = oracle.attn_fwd_rows(q64[b, h], k64[b, h // G], v64[b, h // G], cfg.scale,
                                        cfg.causal, rows)
        og = host(o_g[b, h, rows])
        lg = host(lse_g[b, h, rows])
        o_all.append(og)
        r_all.append(o_r)
        lerr = max(lerr, float(np.abs(lg - l_r).max()))
    err = max_abs_rel(np.stack(o_all), np.stack(r_all))
    return err, lerr


def check_d_rows(cfg, inp, gpu, heads, rows):
    """D = rowsum(dO * O) from the select pass, vs the oracle's exact O, on the
    sampled rows that lie in kept blocks (the pass writes D only there); the
    sampled rows of skipped blocks must hold exact zeros.

    Returns the largest ratio of each row's error to its allowed error: the
    output tolerance (relative to the largest |D| of the sample) plus the
    rounding floor of D's input O, which the path stores in the problem dtype
    -- one unit in the last place of each O element, weighted by |dO|, since a
    sum of products that cancels can lose all of its digits to that rounding.
    A value <= 1 passes."""
    q64, k64, v64, d64 = (to_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    G = cfg.Hq // cfg.Hkv
    rows = np.asarray(rows)
    keep = gpu["sel"]["block_w"].cpu().numpy() != 0
    got, want, floor = [], [], []
    ulp = 2.0 ** -8 if cfg.dtype == "bf16" else 2.0 ** -23
    for b, h in heads:
        kr = keep[b, h, rows // cfg.block]
        d_rows = host(gpu["sel"]["D"][b, h, rows])
        assert np.all(d_rows[~kr] == 0.0), "D of a skipped block's row is not zero"
        if not kr.any():
            continue
        r = rows[kr]
        o_r, _ = oracle.attn_fwd_rows(q64[b, h], k64[b, h // G], v64[b, h // G], cfg.scale,
                                      cfg.causal, r)
        want.append((d64[b, h, r] * o_r).sum(axis=1))
        floor.append(ulp * (np.abs(d64[b, h, r]) * np.abs(o_r)).sum(axis=1))
        got.append(d_rows[kr])
    if not got:
        return 0.0
    got, want, floor = np.concatenate(got), np.concatenate(want), np.concatenate(floor)
    allowed = TOL[cfg.dtype] * np.abs(want).max() + floor
    return float((np.abs(got - want) / allowed).max())


def oracle_bwd_group(cfg, inp, ref_sel, b, g, keep=None):
    """Oracle sparse backward restricted to the query heads of kv group (b, g)."""
    q64, k64, v64, d64 = (to_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    G = cfg.Hq // cfg.Hkv
    heads = [(b, g * G + x) for x in range(G)]
    keep = ref_sel["keep"] if keep is None else keep
    return oracle.attn_bwd_sparse(q64, k64, v64, d64, cfg.block, keep, ref_sel["w"], cfg.scale,
                                  cfg.causal, heads=heads), heads
