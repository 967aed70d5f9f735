#!/usr/bin/env python3
"""Benchmark of LazyFlash-style attention on one MI355X.

A step is one pass of the whole path over one synthetic batch: dense forward
(O, LSE), block selection (masses, D, tau, draw, compaction), sparse backward
(dK/dV walk; dQ plan, walk and finalize), each with a fresh selection seed.  Inputs are
resident in HBM before timing starts.  The headline metric is the attention
backward of one layer -- select + backward, the part the method changes -- as
effective dense-equivalent TFLOP/s (dense backward FLOPs / measured time);
ms per microbatch and the delta sweep ride along.

Prints ONE JSON line on stdout (progress goes to stderr).

    python bench.py [--steps K] [--warmup W] [--config headline] [--delta 0.1]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "dkdv_bf16_kernel_headline_traffic.json")
BWD_SOURCE = os.path.join(ROOT, "block_sparse_backward_amd", "csrc", "lf_bwd.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="headline")
    ap.add_argument("--delta", type=float, default=None, help="main delta (default 0.1)")
    ap.add_argument("--sweep-steps", type=int, default=5,
                    help="steps per extra delta of the sweep (0: no sweep)")
    ap.add_argument("--rule-steps", type=int, default=5,
                    help="steps per selection rule of the equal-kept-fraction comparison (0: skip)")
    ap.add_argument("--train-steps", type=int, default=5,
                    help="timed steps of the autograd training step per delta (0: skip)")
    ap.add_argument("--ceiling-reps", type=int, default=5,
                    help="timed reps of the vendor bf16 GEMM that measures the practical MFMA "
                         "ceiling of this GPU (0: skip)")
    ap.add_argument("--config-steps", type=int, default=3,
                    help="timed steps per delta of each other configuration in the line's "
                         "'configs' array (0: skip them)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0,
                    help="approximate CPU seconds spent on the oracle baseline sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one plain fp32 copy kernel over this many MiB (a known "
                         "byte count that calibrates HBM traffic counters)")
    return ap.parse_args()


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only (the method needs no exchange "
              "between GPUs inside the attention backward); run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_sparse_backward_amd import binding as bd
    from block_sparse_backward_amd import metrics
    from block_sparse_backward_amd.synth import CONFIGS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    bd.load()  # fail loudly if the HIP library is missing
    cfg = CONFIGS[args.config]
    main_delta = args.delta if args.delta is not None else (0.1 if 0.1 in cfg.deltas else cfg.deltas[-1])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)  # reads and writes copy_probe_mib MiB each
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] copy probe: {args.copy_probe_mib} MiB read + written")
    log(f"[bench] generating {cfg}")
    t0 = time.perf_counter()
    inp = make_inputs(cfg, 0)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM ({time.perf_counter() - t0:.1f}s)")

    # preallocated outputs: no allocation inside the timed region
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = bd.bwd_workspace(q, k, cfg.block, cfg.causal)
    stream = torch.cuda.current_stream(dev)

    def run_steps(delta, seeds, split=False):
        """One step per seed: the forwards first, then the backward steps
        (selection, then the backward) back to back, as in a training step
        whose backward pass runs over the layers after the forward pass.  The
        backward is the library's one call, timed with the selection as one
        interval (split=False: columns fwd, select + backward; no event between
        the two, since an event record on the stream delays the next launch by
        a few microseconds), or its dK/dV and dQ phases as two calls, each
        timed (split=True: columns fwd, select, dK/dV, dQ).
        Returns the wall time, per-step times and the selections."""
        sels = [bd.select_outputs(cfg.B, cfg.Hq, cfg.N, cfg.block, dev) for _ in seeds]
        evf = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in seeds]
        evb = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in seeds]
        common = dict(block=cfg.block, causal=cfg.causal, scale=cfg.scale, out=(dq, dk, dv),
                      workspace=ws)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for ev in evf:
            ev[0].record(stream)
            bd.attn_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale, block=cfg.block, out=(o, lse))
            ev[1].record(stream)
        for seed, sel, ev in zip(seeds, sels, evb):
            ev[0].record(stream)
            bd.block_select(o, do, delta, seed, block=cfg.block, causal=cfg.causal,
                            scale=cfg.scale, heads_kv=cfg.Hkv, out=sel)
            if split:
                ev[1].record(stream)
                bd.attn_bwd(q, k, v, lse, do, sel, phases=bd.BWD_DKDV, **common)
                ev[2].record(stream)
                bd.attn_bwd(q, k, v, lse, do, sel, phases=bd.BWD_DQ, **common)
            else:
                bd.attn_bwd(q, k, v, lse, do, sel, phases=bd.BWD_ALL, **common)
            ev[3].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        if split:
            ms = np.array([[f[0].elapsed_time(f[1])] + [e[i].elapsed_time(e[i + 1]) for i in range(3)]
                           for f, e in zip(evf, evb)])
        else:
            ms = np.array([[f[0].elapsed_time(f[1]), e[0].elapsed_time(e[3])]
                           for f, e in zip(evf, evb)])
        flops = [metrics.bwd_flops_kept(s["block_w"].cpu().numpy(), cfg.N, cfg.d, cfg.block,
                                        cfg.causal) for s in sels]
        kept = [float((s["block_w"] != 0).float().mean().item()) for s in sels]
        return wall, ms, np.array(flops, dtype=np.float64), np.array(kept)

    F_dense = metrics.bwd_flops_dense(cfg.B, cfg.Hq, cfg.N, cfg.d, cfg.causal)
    F_fwd = metrics.fwd_flops(cfg.B, cfg.Hq, cfg.N, cfg.d, cfg.causal)

    log(f"[bench] warmup {args.warmup} steps, delta={main_delta}")
    run_steps(main_delta, list(range(10_000, 10_000 + args.warmup)))
    log(f"[bench] timing {args.steps} steps, delta={main_delta}")
    wall, ms, flops, kept = run_steps(main_delta, list(range(args.steps)))
    # columns: fwd, select + backward (one call)
    t_fwd = ms[:, 0].mean()
    per_step_attn = ms[:, 1]
    t_attn_bwd = float(per_step_attn.mean())
    # the same steps with the selection and the backward's two phases timed
    # apart (the dK/dV walk alone is the roofline kernel)
    log(f"[bench] phase breakdown {args.steps} steps, delta={main_delta}")
    _, ms_s, flops_s, _ = run_steps(main_delta, list(range(args.steps)), split=True)
    t_kv, t_q = ms_s[:, 2].mean(), ms_s[:, 3].mean()
    t_sel = float(ms_s[:, 1].mean())
    per_step_bwd = per_step_attn - ms_s[:, 1]  # same seeds in both passes
    t_bwd = float(per_step_bwd.mean())
    value = F_dense / (t_attn_bwd * 1e-3) / 1e12
    log(f"[bench] fwd {t_fwd:.3f} ms, select {t_sel:.3f} ms, bwd {t_bwd:.3f} ms "
        f"(apart: dK/dV {t_kv:.3f}, dQ {t_q:.3f}), kept {kept.mean():.4f}")

    sweep = {}
    for dl in cfg.deltas:
        if dl == main_delta:
            sweep[dl] = (ms, flops, kept, ms_s)
            continue
        if args.sweep_steps <= 0:
            continue
        log(f"[bench] sweep delta={dl}")
        run_steps(dl, [20_000])
        _, ms_d, fl_d, kept_d = run_steps(dl, list(range(args.sweep_steps)))
        _, ms_p, _, _ = run_steps(dl, list(range(args.sweep_steps)), split=True)
        sweep[dl] = (ms_d, fl_d, kept_d, ms_p)
    sweep_out = []
    for dl in sorted(sweep):
        ms_d, fl_d, kept_d, ms_p = sweep[dl]
        attn_ms = float(ms_d[:, 1].mean())
        bwd_d = ms_d[:, 1] - ms_p[:, 1]  # the select timed in the split pass, same seeds
        sweep_out.append(dict(
            delta=dl, steps=int(ms_d.shape[0]), select_ms=round(float(ms_p[:, 1].mean()), 4),
            bwd_ms=round(float(bwd_d.mean()), 4),
            attn_bwd_ms=round(attn_ms, 4),
            attn_bwd_ms_min=round(float(ms_d[:, 1].min()), 4),
            attn_bwd_ms_max=round(float(ms_d[:, 1].max()), 4),
            eff_tflops=round(F_dense / (attn_ms * 1e-3) / 1e12, 2),
            kept_fraction=round(float(kept_d.mean()), 5),
            kept_work_fraction=round(float(fl_d.mean() / F_dense), 5),
            bwd_tflops_on_kept=round(float(fl_d.sum() / (bwd_d.sum() * 1e-3) / 1e12), 2),
            dkdv_ms=round(float(ms_p[:, 2].mean()), 4), dq_ms=round(float(ms_p[:, 3].mean()), 4),
        ))
    dense_ms = next((s["attn_bwd_ms"] for s in sweep_out if s["delta"] == 0.0), None)
    speedup = round(dense_ms / t_attn_bwd, 3) if dense_ms else None

    # Roofline of the dominant kernel, the dK/dV walk (one launch per step,
    # timed alone by the events around its phase in the pass with the phases
    # apart).  Its algorithmic work is
    # four of the five backward products (S, dP, dV, dK: 8 d FLOP) over the
    # unmasked (query, key) pairs of kept blocks, i.e. 0.8 F_kept.  The dQ
    # phase (plan, walk, finalize) recomputes S and dP and adds dS K: 6 d
    # FLOP per pair executed, 2 d of them algorithmic.
    peak = metrics.MI355X_PEAK["bf16_flops"] / 1e12
    f_kv = 0.8 * flops_s
    achieved = float(f_kv.sum() / (ms_s[:, 2].sum() * 1e-3) / 1e12)
    traffic = None
    if os.path.exists(PROFILE_TRAFFIC):
        prof = json.load(open(PROFILE_TRAFFIC))
        if prof.get("source_sha256") == source_sha(BWD_SOURCE) and \
                prof.get("workload") == cfg.name and prof.get("delta") == main_delta:
            traffic = prof.get("bytes_per_launch")
    roofline = dict(bound="mfma", achieved=round(achieved, 2), peak=peak, unit="TFLOP/s",
                    frac=round(achieved / peak, 4), traffic=traffic,
                    kernel="dkdv_bf16_kernel",
                    work_per_unit="8*d FLOP per unmasked (query, key) pair of a kept block",
                    algorithmic_flops_per_launch=float(f_kv.mean()),
                    avg_launch_ms=round(float(t_kv), 4))
    bwd_walks = dict(
        kept_tile_mfma_frac=round(float(flops.sum() / (per_step_bwd.sum() * 1e-3) / 1e12) / peak, 4),
        note="F_kept (10 d FLOP per unmasked kept pair) / t_bwd / peak",
        dq_phase_executed_tflops=round(
            float(0.6 * flops_s.sum() / (ms_s[:, 3].sum() * 1e-3) / 1e12), 2))
    others = dict(
        fwd=dict(bound="mfma", achieved=round(F_fwd / (t_fwd * 1e-3) / 1e12, 2), peak=peak,
                 unit="TFLOP/s"),
        select_mass_pass=dict(bound="hbm",
                              bytes_per_launch=int(q.numel() * q.element_size() * (1.0 + 2.0 * float(kept.mean()))
                                                   + 4 * cfg.B * cfg.Hq * cfg.N),
                              unit="GB/s", peak=8000.0,
                              note="select = mass pass (dO read once) + per-head tau kernel + D "
                                   "pass (dO, O of kept blocks read, D written); time includes "
                                   "all three"),
    )
    others["select_mass_pass"]["achieved_incl_tau"] = round(
        others["select_mass_pass"]["bytes_per_launch"] / (t_sel * 1e-3) / 1e9, 1)

    rules = None
    if args.rule_steps > 0:
        rules = selection_rules_report(cfg, q, k, v, o, lse, do, ws, main_delta,
                                       float(kept.mean()), args.rule_steps)

    training = None
    if args.train_steps > 0:
        training = training_step_report(cfg, q, k, v, do, main_delta, args.train_steps)

    ceiling = None
    if args.ceiling_reps > 0:
        log("[bench] vendor GEMM ceiling")
        ceiling = mfma_ceiling(args.ceiling_reps, peak)
        ceiling["dkdv_vs_ceiling"] = round(achieved / ceiling["achieved"], 4)
        ceiling["fwd_vs_ceiling"] = round(others["fwd"]["achieved"] / ceiling["achieved"], 4)
        # context, not a result: the dK/dV walk on one selection, with the real
        # Q, K, V, dO and with all-zero ones (same kept blocks, same work): the
        # clock the chip holds depends on the data the MFMAs switch
        sel = bd.block_select(o, do, main_delta, 0, block=cfg.block, causal=cfg.causal,
                              scale=cfg.scale, heads_kv=cfg.Hkv)
        zeros = [torch.zeros_like(t) for t in (q, k, v, do)]
        kw = dict(block=cfg.block, causal=cfg.causal, scale=cfg.scale, out=(dq, dk, dv),
                  workspace=ws, phases=bd.BWD_DKDV)

        def dkdv_ms(qq, kk, vv, dd):
            bd.attn_bwd(qq, kk, vv, lse, dd, sel, **kw)
            torch.cuda.synchronize()
            ts = []
            for _ in range(args.ceiling_reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                bd.attn_bwd(qq, kk, vv, lse, dd, sel, **kw)
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            return float(np.median(ts))
        real_ms = dkdv_ms(q, k, v, do)
        zero_ms = dkdv_ms(*zeros)
        del zeros
        ceiling["dkdv_same_selection"] = dict(
            real_operands_ms=round(real_ms, 4), zero_operands_ms=round(zero_ms, 4),
            zero_over_real_speed=round(real_ms / zero_ms, 3),
            note="the dK/dV walk alone, one selection, median of the reps; zero operands are "
                 "context for the clock's data dependence, never a result")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, inp, main_delta, args.cpu_budget_s, metrics)

    # the other workloads, each at its deltas: compact rows (the headline's own
    # deltas are in delta_sweep above)
    others_cfg = None
    if args.config_steps > 0:
        del q, k, v, do, o, lse, dq, dk, dv, ws, inp
        torch.cuda.empty_cache()
        others_cfg = [row for name in ("tiny", "mid", "long", "noncausal") if name != cfg.name
                      for row in config_rows(CONFIGS[name], args.config_steps, peak)]

    out = {
        "metric": f"attention-bwd effective dense-equivalent TFLOP/s (select + sparse bwd, one "
                  f"layer) at N={cfg.N}, delta={main_delta}",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic: seeded N(0,1) Q/K/V, dO with per-row lognormal(0,%g) scale%s; no "
                "model or dataset" % (cfg.sigma, ", %d%% of blocks x%g" % (
                    round(100 * cfg.boost_frac), cfg.boost) if cfg.boost_frac else ""),
        "config": {"workload": f"{cfg.name}: one attention layer, B={cfg.B} Hq={cfg.Hq} "
                               f"Hkv={cfg.Hkv} N={cfg.N} d={cfg.d} block={cfg.block} "
                               f"{'causal' if cfg.causal else 'non-causal'}",
                   "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "N": cfg.N, "d": cfg.d,
                   "block": cfg.block, "causal": cfg.causal, "delta": main_delta},
        "attn_bwd_ms_per_microbatch": round(t_attn_bwd, 4),
        "attn_bwd_ms_min": round(float(per_step_attn.min()), 4),
        "attn_bwd_ms_max": round(float(per_step_attn.max()), 4),
        "select_ms": round(t_sel, 4),
        "bwd_ms": round(t_bwd, 4),
        "bwd_phases_ms": {"dkdv": round(t_kv, 4), "dq": round(t_q, 4)},
        "fwd_ms": round(t_fwd, 4),
        "kept_fraction": round(float(kept.mean()), 5),
        "kept_work_fraction": round(float(flops.mean() / F_dense), 5),
        "speedup_vs_own_dense": speedup,
        "fwd_plus_bwd_speedup_vs_own_dense": (
            round((t_fwd + dense_ms) / (t_fwd + t_attn_bwd), 3) if dense_ms else None),
        "delta_sweep": sweep_out,
        "training_step": training,
        "selection_rules": rules,
        "roofline": roofline,
        "bwd_walks": bwd_walks,
        "other_kernels": others,
        "mfma_ceiling": ceiling,
        "cpu_baseline": cpu,
        "configs": others_cfg,
        "timing": "HIP events on the launch stream, steady state (caches not flushed); the "
                  "steps' forwards run first, then their select+bwd back to back (a training "
                  "step's backward pass follows the whole forward pass); the backward is the "
                  "library's one call (the dQ plan runs alongside the dK/dV walk), timed with "
                  "the selection as one interval (no event between them); select_ms, "
                  "bwd_phases_ms and the roofline come from a second pass over the same seeds "
                  "with the selection and the two phases timed apart, and bwd_ms is the one "
                  "interval less select_ms; ms_per_step is host wall time of the first pass "
                  "per step",
    }
    print(json.dumps(out), flush=True)


def config_rows(cfg, steps, peak):
    """One compact row per delta of workload `cfg`: select + backward (the
    library's one call) per microbatch, effective dense-equivalent TFLOP/s,
    the kept fractions, the dK/dV walk alone (timed in a second pass over
    the same seeds) with its roofline fraction on its algorithmic work
    (0.8 F_kept; bf16 only, the fp32 path does not use the matrix cores), and
    the speedup over the same kernels at delta = 0."""
    import numpy as np
    import torch

    from block_sparse_backward_amd import binding as bd
    from block_sparse_backward_amd import metrics
    from block_sparse_backward_amd.synth import make_inputs

    dev = torch.device("cuda:0")
    log(f"[bench] config {cfg.name}: generating")
    inp = make_inputs(cfg, 0)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
    del inp
    o, lse = bd.attn_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale, block=cfg.block)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = bd.bwd_workspace(q, k, cfg.block, cfg.causal)
    stream = torch.cuda.current_stream(dev)
    common = dict(block=cfg.block, causal=cfg.causal, scale=cfg.scale, out=(dq, dk, dv),
                  workspace=ws)
    F_dense = metrics.bwd_flops_dense(cfg.B, cfg.Hq, cfg.N, cfg.d, cfg.causal)

    def select(delta, seed, sel):
        return bd.block_select(o, do, delta, seed, block=cfg.block, causal=cfg.causal,
                               scale=cfg.scale, heads_kv=cfg.Hkv, out=sel)

    rows = []
    for delta in cfg.deltas:
        log(f"[bench] config {cfg.name} delta={delta}")
        seeds = list(range(steps))
        sels = [bd.select_outputs(cfg.B, cfg.Hq, cfg.N, cfg.block, dev) for _ in seeds]
        select(delta, 30_000, sels[0])
        bd.attn_bwd(q, k, v, lse, do, sels[0], **common)  # warm-up
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in seeds]
        torch.cuda.synchronize()
        for seed, sel, e in zip(seeds, sels, ev):  # select + backward, one call
            e[0].record(stream)
            select(delta, seed, sel)
            bd.attn_bwd(q, k, v, lse, do, sel, **common)
            e[1].record(stream)
        for seed, sel, e in zip(seeds, sels, ev):  # the same seeds, phases apart
            select(delta, seed, sel)
            e[2].record(stream)
            bd.attn_bwd(q, k, v, lse, do, sel, phases=bd.BWD_DKDV, **common)
            e[3].record(stream)
            bd.attn_bwd(q, k, v, lse, do, sel, phases=bd.BWD_DQ, **common)
            e[4].record(stream)
        torch.cuda.synchronize()
        t = np.array([[e[0].elapsed_time(e[1]), e[2].elapsed_time(e[3]), e[3].elapsed_time(e[4])]
                      for e in ev])
        flops = np.array([metrics.bwd_flops_kept(s["block_w"].cpu().numpy(), cfg.N, cfg.d,
                                                 cfg.block, cfg.causal) for s in sels], dtype=float)
        kept = float(np.mean([(s["block_w"] != 0).float().mean().item() for s in sels]))
        row = dict(workload=cfg.name, B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, N=cfg.N, d=cfg.d,
                   block=cfg.block, causal=cfg.causal, dtype=cfg.dtype, delta=delta,
                   steps=steps, attn_bwd_ms=round(float(t[:, 0].mean()), 4),
                   eff_tflops=round(F_dense / (t[:, 0].mean() * 1e-3) / 1e12, 2),
                   kept_fraction=round(kept, 5),
                   kept_work_fraction=round(float(flops.mean() / F_dense), 5),
                   dkdv_ms=round(float(t[:, 1].mean()), 4), dq_ms=round(float(t[:, 2].mean()), 4))
        if cfg.dtype == "bf16":
            dkdv_tf = float(0.8 * flops.sum() / (t[:, 1].sum() * 1e-3) / 1e12)
            row["dkdv_roofline_frac"] = round(dkdv_tf / peak, 4)
        rows.append(row)
    # the same kernels at delta = 0 (every block kept, weight 1): the dense
    # reference each row's speedup is taken against
    dense = [r["attn_bwd_ms"] for r in rows if r["delta"] == 0.0]
    if dense:
        dense_ms = dense[0]
    else:
        log(f"[bench] config {cfg.name} delta=0 (dense reference)")
        sel = bd.select_outputs(cfg.B, cfg.Hq, cfg.N, cfg.block, dev)
        select(0.0, 30_000, sel)
        bd.attn_bwd(q, k, v, lse, do, sel, **common)  # warm-up
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for seed, e in enumerate(ev):
            e[0].record(stream)
            select(0.0, seed, sel)
            bd.attn_bwd(q, k, v, lse, do, sel, **common)
            e[1].record(stream)
        torch.cuda.synchronize()
        dense_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    for r in rows:
        r["dense_attn_bwd_ms"] = round(dense_ms, 4)
        r["speedup_vs_own_dense"] = round(dense_ms / r["attn_bwd_ms"], 3)
    del q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return rows


def mfma_ceiling(reps, peak, n=16384):
    """The bf16 MFMA rate this GPU sustains on a plain large GEMM (the vendor
    library behind torch.matmul, N(0,1) operands), timed like the kernels.
    Sustained MFMA work lowers the clock below the 2.4 GHz of the published
    peak, so this is the practical ceiling the kernels are compared with.  The
    same GEMM on all-zero operands is timed too: the clock the chip holds
    depends on the data the MFMAs switch, and random operands (like the
    kernels' real inputs) hold it lowest."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    a = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)

    def timed(x, y):
        for _ in range(2):
            c = x @ y
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            c = x @ y
        e1.record()
        torch.cuda.synchronize()
        del c
        return e0.elapsed_time(e1) / reps

    ms = timed(a, b)
    z = torch.zeros_like(a)
    ms_zero = timed(z, z)
    del a, b, z
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    tf_zero = 2.0 * n ** 3 / (ms_zero * 1e-3) / 1e12
    return dict(kind=f"torch.matmul bf16 {n}x{n}x{n}, N(0,1) operands (vendor GEMM)", reps=reps,
                ms=round(ms, 4), achieved=round(tf, 2), unit="TFLOP/s",
                frac_of_peak=round(tf / peak, 4),
                zero_operands_tflops=round(tf_zero, 2),
                zero_operands_frac_of_peak=round(tf_zero / peak, 4))


def selection_rules_report(cfg, q, k, v, o, lse, do, ws, delta, kept_frac, steps):
    """The budget against a fixed fraction and top-k at the same kept fraction,
    i.e. at equal backward work (LazyFlash entry, section on block choice).
    Per rule: select + backward time, kept fraction, and the gradient's
    distance to the dense gradient (delta = 0), relative, over dQ, dK, dV:
    per step (the estimator's spread), and of the mean over the steps' draws
    (what stays is bias: a random unbiased draw averages out, top-k drops the
    same blocks every step)."""
    import numpy as np
    import torch

    from block_sparse_backward_amd import binding as bd

    stream = torch.cuda.current_stream()
    common = dict(block=cfg.block, causal=cfg.causal, scale=cfg.scale, workspace=ws)

    def grads(rule, param, seed):
        sel = bd.block_select(o, do, param, seed, block=cfg.block, causal=cfg.causal,
                              scale=cfg.scale, heads_kv=cfg.Hkv, rule=rule)
        return sel, bd.attn_bwd(q, k, v, lse, do, sel, **common)

    _, dense = grads(bd.SELECT_BUDGET, 0.0, 0)
    dense = [x.float() for x in dense]
    dnorm = float(sum((x * x).sum() for x in dense).sqrt())
    out = []
    for name, rule, param in (("budget", bd.SELECT_BUDGET, delta),
                              ("fixed_fraction", bd.SELECT_FRACTION, kept_frac),
                              ("topk", bd.SELECT_TOPK, kept_frac)):
        log(f"[bench] selection rule {name} ({param:.4g})")
        grads(rule, param, 777)  # warm-up
        ms, errs, kept = [], [], []
        acc = [torch.zeros_like(x) for x in dense]
        for s in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            sel, g = grads(rule, param, s)
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
            kept.append(float((sel["block_w"] != 0).float().mean().item()))
            gf = [x.float() for x in g]
            errs.append(float(sum(((a - b) ** 2).sum() for a, b in zip(gf, dense)).sqrt()) / dnorm)
            for a, b in zip(acc, gf):
                a += b
        mean_err = float(sum(((a / steps - b) ** 2).sum() for a, b in zip(acc, dense)).sqrt()) / dnorm
        out.append(dict(rule=name, param=round(float(param), 6), steps=steps,
                        attn_bwd_ms=round(float(np.mean(ms)), 4),
                        kept_fraction=round(float(np.mean(kept)), 5),
                        grad_rel_err_per_step=round(float(np.mean(errs)), 5),
                        grad_rel_err_of_mean=round(mean_err, 5)))
    return {"workload": cfg.name, "note": "equal kept fraction = the budget's mean kept "
            "fraction; errors relative to the dense gradient (delta = 0) over dQ, dK, dV; "
            "attn_bwd_ms = select + backward, events around each step (no other work between)",
            "rules": out}


def training_step_report(cfg, q, k, v, do, delta, steps):
    """One attention layer's training step as a user runs it: the autograd
    wrapper's forward, then o.backward(dO) (selection + sparse backward, a new
    draw seed per step), against the same step at delta = 0 (every block kept:
    the dense backward through the same kernels).  The forward is dense in
    both, which caps the step's speedup at (t_fwd + t_bwd_dense) / t_fwd."""
    import numpy as np
    import torch

    from block_sparse_backward_amd.autograd import draw_seed, lazyflash_attention

    stream = torch.cuda.current_stream()
    leaves = [t.detach().clone().requires_grad_(True) for t in (q, k, v)]

    def run(dl, first_step, n):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        for i in range(n):
            for t in leaves:
                t.grad = None
            ev[i][0].record(stream)
            o = lazyflash_attention(*leaves, dl, draw_seed(first_step + i), causal=cfg.causal,
                                    scale=cfg.scale, block=cfg.block)
            ev[i][1].record(stream)
            o.backward(do)
            ev[i][2].record(stream)
            del o
        torch.cuda.synchronize()
        return np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])] for e in ev])

    res = {}
    for dl in (delta, 0.0):
        log(f"[bench] training step (autograd) delta={dl}")
        run(dl, 1000, 2)
        res[dl] = run(dl, 0, steps).mean(axis=0)
    (f_s, b_s), (f_d, b_d) = res[delta], res[0.0]
    return {"delta": delta, "steps": steps,
            "fwd_ms": round(float(f_s), 4), "bwd_ms": round(float(b_s), 4),
            "step_ms": round(float(f_s + b_s), 4),
            "dense_fwd_ms": round(float(f_d), 4), "dense_bwd_ms": round(float(b_d), 4),
            "dense_step_ms": round(float(f_d + b_d), 4),
            "bwd_speedup": round(float(b_d / b_s), 3),
            "step_speedup": round(float((f_d + b_d) / (f_s + b_s)), 3),
            "amdahl_bound": round(float((f_d + b_d) / f_d), 3),
            "note": "block_sparse_backward_amd.autograd.lazyflash_attention forward + "
                    "o.backward(dO); bwd includes selection; the dense forward bounds the "
                    "step speedup at amdahl_bound"}


def host_description():
    """Cores this process may run on, the CPU model and the BLAS library
    NumPy calls (with its thread count)."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", None
    try:
        import numpy  # noqa: F401  (loads the BLAS that threadpoolctl reports)
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                blas = "%s %s, %s kernels (%s)" % (
                    p.get("internal_api"), p.get("version"), p.get("architecture"),
                    os.path.basename(p.get("filepath", "")))
                threads = p.get("num_threads")
                break
    except Exception:  # pragma: no cover
        pass
    return cores, model, blas, threads


def cpu_baseline(cfg, inp, delta, budget_s, metrics):
    """The oracle, timed on the host cores, in two legs on the same workload:
    selection + sparse backward on whole GQA groups until about `budget_s`
    seconds are spent (the reported value), and the dense backward -- the
    oracle's backward with every block kept at weight 1, i.e. delta = 0 --
    on query blocks of one head until about budget_s / 2 seconds are spent.
    Both are given as dense-equivalent TFLOP/s (the metric's unit) and as the
    time one microbatch would take at that rate."""
    import numpy as np

    import oracle
    from block_sparse_backward_amd.synth import to_f64

    cores, model, blas, blas_threads = host_description()
    G = cfg.Hq // cfg.Hkv
    F_layer = metrics.bwd_flops_dense(cfg.B, cfg.Hq, cfg.N, cfg.d, cfg.causal)
    spent = 0.0
    heads_done = 0
    groups = [(b, g) for b in range(cfg.B) for g in range(cfg.Hkv)]
    log(f"[bench] cpu baseline: oracle on whole GQA groups, ~{budget_s}s budget")
    for b, g in groups:
        hs = slice(g * G, (g + 1) * G)
        q64 = to_f64(inp["q"][b:b + 1, hs])
        d64 = to_f64(inp["dout"][b:b + 1, hs])
        k64 = to_f64(inp["k"][b:b + 1, g:g + 1])
        v64 = to_f64(inp["v"][b:b + 1, g:g + 1])
        t0 = time.perf_counter()
        mass = oracle.block_masses(d64, cfg.block)
        sel = oracle.select(mass, delta, 0)
        oracle.attn_bwd_sparse(q64, k64, v64, d64, cfg.block, sel["keep"], sel["w"], cfg.scale,
                               cfg.causal)
        spent += time.perf_counter() - t0
        heads_done += G
        if spent >= budget_s:
            break
    f_sample = metrics.bwd_flops_dense(1, heads_done, cfg.N, cfg.d, cfg.causal)
    rate = f_sample / spent

    # dense leg: query blocks of head (0, 0) in a seeded random order (the
    # oracle's cost per block does not depend on its position, its causal
    # work does: a spread sample gives the head's average), every one kept
    # with weight 1
    log(f"[bench] cpu baseline: dense oracle backward, ~{budget_s / 2:.0f}s budget")
    q64 = to_f64(inp["q"][0:1, 0:1])
    d64 = to_f64(inp["dout"][0:1, 0:1])
    k64 = to_f64(inp["k"][0:1, 0:1])
    v64 = to_f64(inp["v"][0:1, 0:1])
    nqb = cfg.nqb
    keep = np.zeros((1, 1, nqb), dtype=bool)
    w1 = np.ones((1, 1, nqb), dtype=np.float32)
    d_spent, d_flops, nblk = 0.0, 0, 0
    for i in np.random.Generator(np.random.PCG64(0)).permutation(nqb):
        keep[:] = False
        keep[0, 0, i] = True
        t0 = time.perf_counter()
        oracle.attn_bwd_sparse(q64, k64, v64, d64, cfg.block, keep, w1, cfg.scale, cfg.causal)
        d_spent += time.perf_counter() - t0
        d_flops += metrics.bwd_flops_kept(keep, cfg.N, cfg.d, cfg.block, cfg.causal)
        nblk += 1
        if d_spent >= budget_s / 2:
            break
    d_rate = d_flops / d_spent
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{heads_done} of {cfg.B * cfg.Hq} query heads ({heads_done // G} GQA "
                      f"groups), select + sparse backward at delta={delta}, seed 0, fp64 NumPy; "
                      f"{spent:.1f} s; value = dense-equivalent FLOPs of the sampled heads / time",
            "seconds": round(spent, 2),
            "ms_per_microbatch": round(F_layer / rate * 1e3, 1),
            "dense_bwd": {"value": round(d_rate / 1e12, 6), "unit": "TFLOP/s",
                          "sample": f"{nblk} of {nqb} query blocks of one head (seeded "
                                    f"random order), every block kept with weight 1 "
                                    f"(the oracle's delta = 0 backward); {d_spent:.1f} s",
                          "seconds": round(d_spent, 2),
                          "ms_per_microbatch": round(F_layer / d_rate * 1e3, 1)},
            "cpu_model": model, "blas": blas, "blas_threads": blas_threads,
            "cores_note": "cores = len(os.sched_getaffinity(0)); NumPy's BLAS runs "
                          "blas_threads threads, the rest of the oracle one"}


if __name__ == "__main__":
    main()
