"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Kept sets (mass, tau, block weights, kept_idx, kept_count) must be bit-identical;
O, dQ, dK, dV within max-abs-rel 2e-2 (bf16) / 1e-4 (fp32), LSE within 1e-3 /
1e-5 absolute, D within the output tolerance (on the sampled rows of the
large shapes, plus the rounding floor of D's input O as the forward stored
it: rows where dO and O cancel keep few of D's digits).  Small shapes compare every
element; the full workload shapes compare the whole kept set plus sampled
outputs the oracle computes exactly (one GQA group)."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_backward_amd.synth import CONFIGS, Config, make_inputs, to_f64
from tests.parity_helpers import (LSE_TOL, TOL, check_d_rows, check_fwd_rows,
                                  check_select_exact, host, max_abs_rel, run_gpu)

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny_f32": (CONFIGS["tiny"], 0.1),
    "bf16_gqa_d128_b128": (Config("s1", 1, 4, 2, 512, 128, "bf16", True, 128, 1.5), 0.1),
    "bf16_dense_delta0": (Config("s2", 1, 4, 2, 512, 128, "bf16", True, 128, 1.5), 0.0),
    "bf16_ragged_d64_b64": (Config("s3", 2, 4, 1, 448, 64, "bf16", True, 64, 1.0), 0.2),
    "bf16_noncausal_d64": (Config("s4", 2, 2, 2, 384, 64, "bf16", False, 64, 0.5), 0.1),
    "bf16_d128_b64_ragged": (Config("s5", 1, 2, 1, 320, 128, "bf16", True, 64, 1.5), 0.1),
    "bf16_gqa8_d64_b128": (Config("s6", 1, 8, 1, 512, 64, "bf16", True, 128, 1.5), 0.05),
    "bf16_noncausal_d128_b128": (Config("s7", 1, 4, 4, 256, 128, "bf16", False, 128, 1.0), 0.3),
    "f32_noncausal_d128": (Config("s8", 1, 2, 1, 128, 128, "f32", False, 64, 1.0), 0.2),
    "bf16_boosted_heavy": (Config("s9", 1, 4, 2, 1024, 128, "bf16", True, 128, 2.0,
                                  boost_frac=0.1, boost=20.0), 0.1),
    # N not a multiple of the block: a partial last query block and key tile
    "bf16_ragged_N1000_b128": (Config("r1", 1, 4, 2, 1000, 128, "bf16", True, 128, 1.5), 0.1),
    "bf16_ragged_N777_noncausal_d64": (Config("r2", 2, 2, 1, 777, 64, "bf16", False, 64, 1.0), 0.2),
    "bf16_ragged_N1100_d64_b128_gqa4": (Config("r3", 1, 8, 2, 1100, 64, "bf16", True, 128, 2.0,
                                               boost_frac=0.2, boost=20.0), 0.05),
    "bf16_ragged_N333_noncausal_d128_b64": (Config("r4", 1, 2, 2, 333, 128, "bf16", False, 64, 0.5),
                                            0.0),
    "f32_ragged_N300": (Config("r5", 1, 2, 2, 300, 64, "f32", True, 64, 1.0), 0.1),
    # fewer rows than one sub-tile: one partial block, one partial key tile
    "bf16_N50_causal_d128_b128": (Config("e1", 1, 4, 2, 50, 128, "bf16", True, 128, 1.5), 0.1),
    "bf16_N1_causal_d64_b64": (Config("e2", 2, 2, 1, 1, 64, "bf16", True, 64, 1.0), 0.0),
    # batch x kv heads a multiple of 8: the workgroup-to-XCD mappings of the
    # forward and the dK/dV walk take their rotated path (B > 1 included)
    "bf16_xcd_B2_Hkv4": (Config("x1", 2, 8, 4, 640, 128, "bf16", True, 128, 2.0,
                                boost_frac=0.1, boost=20.0), 0.1),
    "bf16_xcd_B3_Hkv8_d64_b64": (Config("x2", 3, 8, 8, 384, 64, "bf16", True, 64, 1.5), 0.1),
    # odd group sizes: 3 and 5 query heads per kv head (the walks over a
    # group's heads and the head-to-group maps)
    "bf16_gqa3_d128_b64": (Config("g3", 1, 6, 2, 448, 128, "bf16", True, 64, 1.5,
                                  boost_frac=0.2, boost=20.0), 0.1),
    "bf16_gqa5_noncausal_d64_b128_ragged": (Config("g5", 2, 5, 1, 333, 64, "bf16", False, 128,
                                                   1.0), 0.2),
    "bf16_gqa3_B2_Hkv4_d128_b128_ragged": (Config("g3x", 2, 12, 4, 700, 128, "bf16", True, 128,
                                                  2.0), 0.1),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_parity(name):
    cfg, delta = SMALL[name]
    print(f"[parity] {name} {cfg} delta={delta}", flush=True)
    _check_full(cfg, make_inputs(cfg, 0), delta, seed=0, tag=name)


def _check_full(cfg, inp, delta, seed, tag):
    """Every element of O, LSE, D (kept rows), dQ, dK, dV against the oracle."""
    gpu = run_gpu(cfg, inp, delta, seed=seed)
    ref_sel = check_select_exact(cfg, inp, gpu, delta, seed)
    q64, k64, v64, d64 = (to_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    o_ref, lse_ref = oracle.attn_fwd(q64, k64, v64, cfg.scale, cfg.causal)
    tol = TOL[cfg.dtype]
    assert max_abs_rel(host(gpu["o"]), o_ref) <= tol
    assert np.abs(host(gpu["lse"]) - lse_ref).max() <= LSE_TOL[cfg.dtype]
    # D of the rows of kept blocks (the backward reads no other); the rows of
    # skipped blocks are written as zeros
    d_ref = (d64 * o_ref).sum(axis=-1)
    d_gpu = host(gpu["sel"]["D"])
    kept_rows = np.repeat(ref_sel["keep"], cfg.block, axis=2)[:, :, :cfg.N]
    if kept_rows.any():
        assert max_abs_rel(d_gpu[kept_rows], d_ref[kept_rows]) <= tol
    assert np.all(d_gpu[~kept_rows] == 0.0)
    dq, dk, dv = oracle.attn_bwd_sparse(q64, k64, v64, d64, cfg.block, ref_sel["keep"],
                                        ref_sel["w"], cfg.scale, cfg.causal, o=o_ref, lse=lse_ref)
    errs = [max_abs_rel(host(gpu[n]), r) for n, r in (("dq", dq), ("dk", dk), ("dv", dv))]
    print(f"[parity] {tag} kept={ref_sel['keep'].mean():.3f} errs={errs}", flush=True)
    assert max(errs) <= tol, errs
    # rows of skipped blocks of dq are exact zeros
    skipped = np.repeat(~ref_sel["keep"], cfg.block, axis=2)[:, :, :cfg.N]
    assert np.all(host(gpu["dq"])[skipped] == 0.0)
    return ref_sel


# Causal heads that keep more than 64 blocks: the dK/dV walk holds a head's
# kept list 64 entries at a time in a register, so these walks reload it in
# mid-walk (key tile 0 walks 96 or 128 blocks per head) and the later key
# tiles find their first block past the first 64 entries.  Every element is
# compared, for 128- and 64-row blocks and both head dims.
LONG_WALKS = {
    "causal_96_blocks_per_head_d128_b128": Config("w1", 1, 2, 1, 96 * 128, 128, "bf16", True,
                                                   128, 1.5),
    "causal_128_blocks_per_head_d128_b64": Config("w2", 1, 2, 1, 128 * 64, 128, "bf16", True,
                                                   64, 1.5),
    "causal_130_blocks_per_head_d64_b64_ragged": Config("w3", 1, 4, 2, 130 * 64 - 20, 64, "bf16",
                                                         True, 64, 1.0),
}


@pytest.mark.parametrize("name", list(LONG_WALKS))
def test_long_causal_walk_parity(name):
    cfg = LONG_WALKS[name]
    print(f"[parity-walk] {name} {cfg} delta=0", flush=True)
    ref_sel = _check_full(cfg, make_inputs(cfg, 0), 0.0, seed=0, tag=name)
    assert ref_sel["kept_count"].min() > 64


# Softmax scales other than 1/sqrt(d): a negative scale (the forward negates Q
# so that the running max is taken over the scaled scores), a small one and a
# sharp one; the selection does not depend on the scale, D and the gradients do.
SCALES = {
    "bf16_causal_d128_neg": (Config("c1", 1, 4, 2, 384, 128, "bf16", True, 128, 1.5), -0.09, 0.1),
    "bf16_noncausal_d64_small": (Config("c2", 2, 2, 2, 256, 64, "bf16", False, 64, 1.0), 0.03, 0.2),
    "bf16_causal_d64_b128_sharp": (Config("c3", 1, 4, 1, 320, 64, "bf16", True, 128, 1.0), 0.5, 0.1),
    "f32_causal_d64_neg": (Config("c4", 1, 2, 1, 192, 64, "f32", True, 64, 1.0), -0.2, 0.1),
}


@pytest.mark.parametrize("name", list(SCALES))
def test_softmax_scale_parity(name):
    cfg, scale, delta = SCALES[name]
    print(f"[parity-scale] {name} {cfg} scale={scale} delta={delta}", flush=True)
    inp = make_inputs(cfg, 3)
    gpu = run_gpu(cfg, inp, delta, seed=5, scale=scale)
    ref_sel = check_select_exact(cfg, inp, gpu, delta, 5)
    q64, k64, v64, d64 = (to_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    o_ref, lse_ref = oracle.attn_fwd(q64, k64, v64, scale, cfg.causal)
    tol = TOL[cfg.dtype]
    assert max_abs_rel(host(gpu["o"]), o_ref) <= tol
    assert np.abs(host(gpu["lse"]) - lse_ref).max() <= LSE_TOL[cfg.dtype]
    dq, dk, dv = oracle.attn_bwd_sparse(q64, k64, v64, d64, cfg.block, ref_sel["keep"],
                                        ref_sel["w"], scale, cfg.causal)
    errs = [max_abs_rel(host(gpu[n]), r) for n, r in (("dq", dq), ("dk", dk), ("dv", dv))]
    print(f"[parity-scale] {name} kept={ref_sel['keep'].mean():.3f} errs={errs}", flush=True)
    assert max(errs) <= tol, errs


_CACHE = {}


def _full_inputs(name):
    if name not in _CACHE:
        _CACHE.clear()
        cfg = CONFIGS[name]
        inp = make_inputs(cfg, 0)
        _CACHE[name] = (cfg, inp)
    return _CACHE[name]


FULL = [(n, dl) for n in ("mid", "headline", "long", "noncausal") for dl in CONFIGS[n].deltas]
# Whole-group comparisons (every key of dK/dV, every kept block of dQ) where
# the oracle finishes in tens of seconds: one GQA group of mid at every delta
# and of the headline at delta 0.1 and 0.2 (about 45 and 30 kept blocks of
# 32768-key rows).  The headline at delta 0 (1024 kept blocks in the group)
# and the long shape (about 800) compare the tail keys that only the sampled
# blocks reach, plus the size-free invariants; their walks take the same code
# paths as the whole-group and long-walk cases.
WHOLE_GROUP = {("mid", 0.0), ("mid", 0.05), ("mid", 0.1), ("headline", 0.1), ("headline", 0.2)}


@pytest.mark.parametrize("name,delta", FULL)
def test_full_size_parity(name, delta):
    cfg, inp = _full_inputs(name)
    print(f"[parity-full] {name} delta={delta}", flush=True)
    _check_large(cfg, inp, delta, whole_group=(name, delta) in WHOLE_GROUP)


# The largest supported block count per head (4096) with 64-row blocks:
# N = 262144.  With the headline's dO distribution one head keeps ~140 blocks,
# so the dQ plan cuts them into long chunks (~290 key steps) queued longest
# first; four heads on one kv head with a milder dO keep ~60% of their blocks
# and take the unchunked path.  Both walk the kept list in many 64-entry
# chunks.
MAXBLK = {
    "maxblk_1head_chunked": Config("maxblk1", 1, 1, 1, 4096 * 64, 64, "bf16", True, 64, 2.0,
                                   boost_frac=0.05, boost=20.0),
    "maxblk_gqa4": Config("maxblk4", 1, 4, 1, 4096 * 64, 64, "bf16", True, 64, 1.5),
    # a long ragged length: 4096 blocks of 64 rows, the last with 27
    "maxblk_ragged": Config("maxblkr", 1, 2, 1, 4095 * 64 + 27, 64, "bf16", True, 64, 2.0,
                            boost_frac=0.05, boost=20.0),
    "headline_ragged": Config("headr", 1, 8, 2, 32768 - 77, 128, "bf16", True, 128, 2.0,
                              boost_frac=0.05, boost=20.0),
}


@pytest.mark.parametrize("name", list(MAXBLK))
def test_max_block_count_parity(name):
    cfg = MAXBLK[name]
    print(f"[parity-max] {name} {cfg}", flush=True)
    inp = make_inputs(cfg, 0)
    _check_large(cfg, inp, 0.1)


def _check_large(cfg, inp, delta, whole_group=False):
    name = cfg.name
    gpu = run_gpu(cfg, inp, delta, seed=0)
    ref_sel = check_select_exact(cfg, inp, gpu, delta, 0)
    kept_frac = float(ref_sel["keep"].mean())
    G = cfg.Hq // cfg.Hkv
    b, g = cfg.B - 1, cfg.Hkv // 2
    heads = [(b, g * G + x) for x in range(G)]
    rng = np.random.Generator(np.random.PCG64(1))
    rows = np.unique(np.concatenate([[0, 1, cfg.N - 1], rng.integers(0, cfg.N, 60)]))
    err_o, err_l = check_fwd_rows(cfg, inp, gpu, heads[:2], rows)
    assert err_o <= TOL[cfg.dtype] and err_l <= LSE_TOL[cfg.dtype], (err_o, err_l)
    # D is written for kept blocks only: sample rows of the first kept blocks too
    kept_blocks = np.unique(np.concatenate(
        [np.nonzero(ref_sel["keep"][hb, hh])[0][:3] for hb, hh in heads[:2]]))
    d_rows = np.unique(np.concatenate(
        [rows] + [np.minimum(cfg.N - 1, i * cfg.block + np.array([0, cfg.block // 2, cfg.block - 1]))
                  for i in kept_blocks]))
    assert check_d_rows(cfg, inp, gpu, heads[:2], d_rows) <= 1.0

    q64, k64, v64, d64 = (to_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    keep = ref_sel["keep"]
    nqb = cfg.nqb
    if cfg.causal and not whole_group:
        # dQ of sampled kept blocks (each block's dq depends on that block
        # only), and dK/dV of the keys at and after block jt: under the causal
        # mask only query blocks >= jt reach them, and all of those that are
        # kept are in the sample.  jt is chosen so that about six kept blocks
        # of the group lie at or after it.
        kept_all = sorted({int(i) for bb, h in heads for i in np.nonzero(keep[bb, h])[0]})
        jt = kept_all[-min(6, len(kept_all))] if kept_all else nqb - 1
        sample = np.zeros_like(keep)
        for bb, h in heads:
            kept = np.nonzero(keep[bb, h])[0]
            pick = set(rng.choice(kept, min(3, kept.size), replace=False).tolist())
            pick |= {int(i) for i in kept if i >= jt}
            for i in pick:
                sample[bb, h, i] = True
        dq, dk, dv = oracle.attn_bwd_sparse(q64, k64, v64, d64, cfg.block, sample, ref_sel["w"],
                                            cfg.scale, cfg.causal, heads=heads)
        sel_rows = []
        for bb, h in heads:
            for i in np.nonzero(sample[bb, h])[0]:
                sel_rows.append((bb, h, i))
        got = np.stack([host(gpu["dq"][bb, h, i * cfg.block:(i + 1) * cfg.block])
                        for bb, h, i in sel_rows])
        want = np.stack([dq[bb, h, i * cfg.block:(i + 1) * cfg.block] for bb, h, i in sel_rows])
        e_dq = max_abs_rel(got, want)
        tail = slice(jt * cfg.block, cfg.N)
        assert np.abs(dk[b, g, tail]).max() > 0
        e_dk = max_abs_rel(host(gpu["dk"][b, g, tail]), dk[b, g, tail])
        e_dv = max_abs_rel(host(gpu["dv"][b, g, tail]), dv[b, g, tail])
    else:
        # the whole group: dK/dV of every key, dQ of every row of its heads
        # (the rows of skipped blocks are exact zeros on both sides)
        dq, dk, dv = oracle.attn_bwd_sparse(q64, k64, v64, d64, cfg.block, keep, ref_sel["w"],
                                            cfg.scale, cfg.causal, heads=heads)
        hs = [h for _, h in heads]
        dq_gpu = host(gpu["dq"][b, hs])
        e_dq = max_abs_rel(dq_gpu, dq[b, hs])
        skipped = np.repeat(~keep[b, hs], cfg.block, axis=1)[:, :cfg.N]
        assert np.all(dq_gpu[skipped] == 0.0)
        e_dk = max_abs_rel(host(gpu["dk"][b, g]), dk[b, g])
        e_dv = max_abs_rel(host(gpu["dv"][b, g]), dv[b, g])
    print(f"[parity-full] {name} delta={delta} kept={kept_frac:.4f} fwd={err_o:.2e} "
          f"dq={e_dq:.2e} dk={e_dk:.2e} dv={e_dv:.2e}", flush=True)
    assert max(e_dq, e_dk, e_dv) <= TOL[cfg.dtype]
    # any size: each row of dS sums to zero, so the keys' dK sum to zero; the
    # keys' dV sum to the weighted kept dO rows (per kv head, all query heads)
    dk_all = host(gpu["dk"]).sum(axis=2)
    dv_all = host(gpu["dv"]).sum(axis=2)
    wrow = np.repeat(ref_sel["keep"] * ref_sel["w"].astype(np.float64), cfg.block,
                     axis=2)[:, :, :cfg.N]
    want_dv = (d64 * wrow[..., None]).sum(axis=2).reshape(cfg.B, cfg.Hkv, G, cfg.d).sum(axis=2)
    scale_dk = np.abs(host(gpu["dk"])).max() * np.sqrt(cfg.N)
    assert np.abs(dk_all).max() <= 2e-2 * scale_dk
    assert max_abs_rel(dv_all, want_dv) <= 2e-2
    torch.cuda.empty_cache()
