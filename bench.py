#!/usr/bin/env python3
"""Benchmark of the adaptive-precision attention prefill hot path on one GPU.

One step = the whole path on one batch of resident synthetic inputs:
apa_quantize -> apa_pass1 -> apa_pass2 (fused merge).  The default workload
is the long-context 3B-shaped prefill: B=1, 24 query heads over 8 KV heads,
head dim 128, 2048 query rows aligned to the tail of 122880 keys, causal, fp16,
eps = 0.005.  Prints one JSON line (see --help for the flags).

Throughput is effective TFLOP/s: 4*D*(visible (row, key) pairs) per step over
the step time, the same numerator for APA and the all-exact path.  The
roofline object is for pass 1 (the dominant kernel): its algorithmic FP4 MFMA
work per launch over its average launch time, against the dense FP4 peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP4_TFLOPS = 10100.0      # MI355X dense MXFP4
PEAK_FP16_TFLOPS = 2500.0      # MI355X dense FP16
METRIC = "ms & effective TFLOP/s, causal GQA prefill 2048q×122880k; % of MFMA peak"


def visible_pairs(Nq, Nkv, causal=True):
    if not causal:
        return Nq * Nkv
    off = Nkv - Nq
    r = np.arange(Nq, dtype=np.int64)
    return int(np.minimum(r + off + 1, Nkv).sum())


def cell_counts(hot, Nq, Nkv, causal=True):
    """Visited (group, tile) cells and their (row, key) pairs at tile
    granularity, split into hot and cold, from the hot mask [B,Hq,NG,NT]."""
    NG, NT = hot.shape[-2], hot.shape[-1]
    off = Nkv - Nq
    vis = np.zeros((NG, NT), bool)
    rows = np.zeros(NG, np.int64)
    for g in range(NG):
        last = min(16 * g + 15, Nq - 1)
        d = min(Nkv - 1, last + off) // 64 if causal else NT - 1
        vis[g, :d + 1] = True
        rows[g] = last - 16 * g + 1
    visb = np.broadcast_to(vis, hot.shape)
    pairs = np.broadcast_to((rows[:, None] * 64) * np.ones(NT, np.int64), hot.shape)
    cells = int(visb.sum())
    hot_cells = int((hot & visb).sum())
    vp = int(pairs[visb].sum())
    hp = int(pairs[hot & visb].sum())
    return cells, hot_cells, vp, hp


def src_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mixed_precision_long_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_src, units):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(units)
    if not e or e.get("src_hash") != src_hash(kernel_src):
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def sample_groups(w, ngroups):
    """The row groups the CPU legs use: a seeded random sample of the
    workload's (batch, query head, 16-row group) triples."""
    from oracle import oracle as O
    p = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale=w.scale, eps=w.eps)
    allg = O.all_groups(p)
    return allg[np.random.default_rng(123).choice(len(allg), ngroups, replace=False)]


def cpu_legs(w, eps, ngroups, threads, gpu_out, gpu_hot, exact_out):
    """The oracle as it stands, timed on a bounded sample of row groups of the
    same workload (pass 1, exact pass 2 and merge; the K/V quantisation it
    needs is shared by every row of a KV head and is excluded), and, untimed,
    the FP64 reports on the same rows: the GPU's APA output and the all-exact
    output against FP64 attention, and the true FP64 share of the tiles the
    GPU left cold."""
    from oracle import oracle as O
    from mixed_precision_long_amd.inputs import make_inputs
    p = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale=w.scale, eps=eps)
    sel = sample_groups(w, ngroups)
    kvh = sorted({(int(b), int(h) // (w.Hq // w.Hkv)) for b, h, _ in sel})
    Q, K, V = make_inputs(w, kv_heads=kvh)
    prep = O.quantize(p, Q, K, V)
    t0 = time.perf_counter()
    r = O.run(p, Q, K, V, prep, groups=sel, nthreads=threads)
    dt = time.perf_counter() - t0
    off = w.Nkv - w.Nq
    flops = 0
    for _, _, g in sel:
        for row in range(16 * g, min(16 * g + 16, w.Nq)):
            flops += 4 * w.D * min(row + off + 1, w.Nkv)
    base = dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s (effective)", cores=threads,
                kind="oracle", seconds=round(dt, 2), cpu_model=cpu_model(),
                logical_cores_visible=os.cpu_count(),
                sample="%d random 16-row groups of %s (pass 1 + exact pass 2 + merge; K/V "
                       "quantisation excluded), one worker thread per core of the %d-core "
                       "share a GPU gets on this host" % (ngroups, w.name, threads))
    rows = np.array([(b, h, g * 16 + i) for b, h, g in sel for i in range(16)
                     if g * 16 + i < w.Nq], np.int32)
    rep = O.reports(p, Q, K, V, gpu_hot, rows, nthreads=threads)
    ix = (rows[:, 0], rows[:, 1], rows[:, 2])
    # the GPU's verdicts against the oracle's on the sampled groups: agreement
    # over visited cells and the largest |margin| of a disagreeing one
    vis_c, mism_c, worst_m = 0, 0, 0.0
    for b, h, g in sel:
        mg = r["margin"][b, h, g]
        vis = ~np.isnan(mg)
        diff = vis & (gpu_hot[b, h, g].astype(bool) != r["hot"][b, h, g].astype(bool))
        vis_c += int(vis.sum())
        mism_c += int(diff.sum())
        if diff.any():
            worst_m = max(worst_m, float(np.abs(mg[diff]).max()))
    # the sink as realised: the mass of keys 0..3 (exact softmax) and their
    # mean logit above the row's mean visible logit (nats; the mean key of the
    # visible prefix from prefix sums of K)
    G = w.Hq // w.Hkv
    lift, mass = [], []
    for b, hk in kvh:
        Kh = K[b, hk].astype(np.float64)
        pre = np.cumsum(Kh, axis=0)
        ksink = Kh[:4].mean(axis=0)
        for i in np.flatnonzero((rows[:, 0] == b) & (rows[:, 1] // G == hk)):
            qr = Q[b, rows[i, 1], rows[i, 2]].astype(np.float64)
            last = min(w.Nkv - 1, int(rows[i, 2]) + off)
            s4 = w.scale * (Kh[:4] @ qr)
            mass.append(float(np.exp(s4 - rep["lse"][i]).sum()))
            lift.append(float(w.scale * (qr @ ksink - qr @ (pre[last] / (last + 1)))))
    pct = lambda a, qs: {"p%d" % q: round(float(np.percentile(a, q)), 4) for q in qs}

    def summ(out):
        c = O.compare_rows(out[ix], rep["O_ref"])
        return {"cos_min": round(float(c["cos"].min()), 6),
                "cos_median": round(float(np.median(c["cos"])), 6),
                "mse": float("%.4g" % c["mse"]), "max_abs": round(c["max_abs"], 6)}

    apa = O.compare_rows(gpu_out[ix], rep["O_ref"])
    worst = int(np.argmin(apa["cos"]))
    nref = np.linalg.norm(rep["O_ref"][worst])
    vs = {"rows": len(rows), "sample": "the rows of the CPU baseline's row groups",
          "apa": summ(gpu_out), "oracle_apa": summ(r["O"]),
          "cold_tile_true_share_max": round(float(rep["cold_tile_max"].max()), 6),
          "page_cold_tile_true_share_max": 0.0118,
          "cold_share": {"max": round(float(rep["cold_share"].max()), 6),
                         "median": round(float(np.median(rep["cold_share"])), 6)},
          "worst_row": {"row": [int(x) for x in rows[worst]],
                        "cos": round(float(apa["cos"][worst]), 6),
                        "cold_share": round(float(rep["cold_share"][worst]), 6),
                        "cold_part_norm_over_ref": round(float(
                            np.linalg.norm(rep["O_cold"][worst]) / nref), 6) if nref > 0 else None,
                        "hot_part_norm_over_ref": round(float(
                            np.linalg.norm(rep["O_hot"][worst]) / nref), 6) if nref > 0 else None}}
    if exact_out is not None:
        vs["exact"] = summ(exact_out)
    vs["mask_vs_oracle"] = {"cells": vis_c, "agree": round(1.0 - mism_c / max(vis_c, 1), 6),
                            "mismatches": mism_c, "worst_mismatch_margin": worst_m}
    vs["sink"] = {"keys": 4, "mass": pct(mass, (10, 50, 90)),
                  "lift_nats": pct(lift, (10, 50, 90)), "generator_lift_nats": w.delta}
    return base, vs


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first; the GPU clocks settle over the first ~20 steps")
    ap.add_argument("--workload", default="long3b")
    ap.add_argument("--eps", type=float, default=None)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-exact", action="store_true", help="skip timing the all-exact path")
    ap.add_argument("--cpu-groups", type=int, default=384,
                    help="row groups of the CPU oracle's sample (also the rows of vs_fp64)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the eps sweep")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip timing the accuracy variants (two-term Q, least-squares K scales)")
    ap.add_argument("--no-window", action="store_true",
                    help="skip timing the sliding-window variant (4096 keys)")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip timing the single persistent launch of both passes")
    ap.add_argument("--no-ring", action="store_true",
                    help="skip timing the KV window ring (sink tile + two halves of 96 tiles)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="before warmup, run one plain device-to-device copy of MIB MiB (a "
                         "known-size kernel that scales the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the path is single-GPU by design (it would shard by "
              "(batch, kv-head) with no exchange); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from mixed_precision_long_amd import apa
    from mixed_precision_long_amd.inputs import WORKLOADS, make_inputs, outlier_value_tiles

    w = WORKLOADS[args.workload]
    eps = w.eps if args.eps is None else args.eps
    torch.cuda.set_device(0)
    print("[bench] generating %s inputs" % w.name, file=sys.stderr, flush=True)
    Q, K, V = make_inputs(w)
    data_sha = {n: hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()
                for n, x in (("Q", Q), ("K", K), ("V", V))}
    dt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
    q = torch.from_numpy(Q).to(dt).cuda()
    k = torch.from_numpy(K).to(dt).cuda()
    v = torch.from_numpy(V).to(dt).cuda()
    V_host = V  # kept for the outlier-value inputs of the weighted hot test
    del Q, K
    p = apa.problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D,
                    dtype=apa.APA_F16 if w.dtype == "fp16" else apa.APA_BF16, scale=w.scale)
    bufs = apa.alloc(p)
    stream = torch.cuda.current_stream()

    ev = {n: [] for n in ("quantize", "pass1", "pass2")}

    def step(record):
        if record:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record(stream)
        apa.quantize(p, q, k, v, bufs.fp4, bufs.ws_q, stream)
        if record:
            e[1].record(stream)
        apa.pass1(p, bufs.fp4, eps, bufs.cold_m, bufs.cold_l, bufs.cold_o, bufs.bits, None,
                  ws=bufs.ws_p1, stream=stream)
        if record:
            e[2].record(stream)
        apa.pass2(p, q, k, v, bufs.fp4, bufs.bits, bufs.cold_m, bufs.cold_l, bufs.cold_o, True,
                  out=bufs.out, lse=bufs.lse, ws=bufs.ws_p2, stream=stream)
        if record:
            e[3].record(stream)
            ev["quantize"].append((e[0], e[1]))
            ev["pass1"].append((e[1], e[2]))
            ev["pass2"].append((e[2], e[3]))

    if args.copy_calib > 0:
        n = args.copy_calib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print("[bench] copied %d MiB" % args.copy_calib, file=sys.stderr, flush=True)

    print("[bench] warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    kern_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in ev}
    print("[bench] APA %.3f ms/step %s" % (ms, kern_ms), file=sys.stderr, flush=True)
    gpu_out_host = bufs.out.float().cpu().numpy()

    flop = 4.0 * w.D * visible_pairs(w.Nq, w.Nkv) * w.Hq * w.B
    hot = apa_hot_mask(p, bufs.bits)
    gpu_hot_host = hot.astype(np.uint8)
    cells, hot_cells, vpairs, hpairs = cell_counts(hot, w.Nq, w.Nkv)
    cold_pairs = (vpairs - hpairs) * 1.0
    # pass-1 algorithmic FP4 work per launch: QK on every visited pair, the
    # one-column row sum, PV on the cold pairs (tile granularity)
    w4 = 2.0 * w.D * vpairs + 2.0 * vpairs + 2.0 * w.D * cold_pairs
    w16 = 4.0 * w.D * hpairs
    p1_tflops = w4 / (kern_ms["pass1"] * 1e-3) / 1e12
    t_roof_ms = (w4 / (PEAK_FP4_TFLOPS * 1e12) + w16 / (PEAK_FP16_TFLOPS * 1e12)) * 1e3
    out = bufs.out.float()

    res = {
        "metric": METRIC,
        "value": round(flop / (ms * 1e-3) / 1e12, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4+fp16", "data": "synthetic",
        "config": {"workload": "%s: B%d Hq%d Hkv%d D%d Nq%d Nkv%d causal %s eps %g" % (
            w.name, w.B, w.Hq, w.Hkv, w.D, w.Nq, w.Nkv, w.dtype, eps),
            "global_batch": w.B, "seq_len": w.Nkv, "parallelism": "single-gpu"},
        "kernels_ms": {k2: round(v2, 4) for k2, v2 in kern_ms.items()},
        # the attention alone, with K/V already in the FP4 format (a persistent FP4
        # K/V cache): pass 1 + pass 2 of the same steps
        "apa_attn_ms": round(kern_ms["pass1"] + kern_ms["pass2"], 4),
        "roofline": {"bound": "mfma", "kernel": "k_pass1",
                     "achieved": round(p1_tflops, 3), "peak": PEAK_FP4_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(p1_tflops / PEAK_FP4_TFLOPS, 5),
                     "traffic": traffic_for(["pass1.hip", "pass1_core.h", "apa_device.h", "apa_kernels.h"], "k_pass1"),
                     "algorithmic_fp4_flop_per_launch": w4},
        "weighted_roofline": {"t_roof_ms": round(t_roof_ms, 4),
                              "frac": round(t_roof_ms / ms, 4),
                              "fp4_flop": w4, "fp16_flop": w16},
        "hot_fraction": {"cells": round(hot_cells / max(cells, 1), 5),
                         "pairs": round(hpairs / max(vpairs, 1), 5),
                         "page_real_dumps": "6-10 %"},
        "data_sha256": data_sha,
    }

    exact_out_host = None
    if not args.no_exact:
        eo = torch.empty_like(q)
        el = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
        for _ in range(args.warmup):
            apa.exact(p, q, k, v, eo, el, stream=stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n_ex = max(3, args.steps // 2)
        for _ in range(n_ex):
            apa.exact(p, q, k, v, eo, el, stream=stream)
        torch.cuda.synchronize()
        ems = (time.perf_counter() - t0) * 1e3 / n_ex
        ef = eo.float()
        exact_out_host = ef.cpu().numpy()
        cos = torch.nn.functional.cosine_similarity(out.reshape(-1, w.D), ef.reshape(-1, w.D), dim=1)
        res["exact"] = {"ms": round(ems, 4), "tflops": round(flop / (ems * 1e-3) / 1e12, 3),
                        "fp16_roofline_frac": round(flop / (ems * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 4),
                        "apa_speedup": round(ems / ms, 3)}
        res["apa_vs_exact"] = {"cos_min": round(float(cos.min()), 6),
                               "cos_median": round(float(cos.median()), 6),
                               "max_abs": round(float((out - ef).abs().max()), 5)}
        print("[bench] exact %.3f ms" % ems, file=sys.stderr, flush=True)

    def variant(p2, vv=None, ref=None):
        """One APA configuration on the same inputs (V replaced by vv if
        given): 10 timed steps after 20 (the clocks settle again after the
        all-exact launches), per-kernel times, hot cells, and its output
        against `ref` (the exact output of the same inputs)."""
        vv = v if vv is None else vv
        b2 = apa.alloc(p2)
        ev2 = []
        for i in range(20 + 10):
            step_eps(apa, p2, q, k, vv, b2, eps, stream, ev2 if i >= 20 else None)
        torch.cuda.synchronize()
        hot2 = apa_hot_mask(p2, b2.bits)
        c2, h2, _, _ = cell_counts(hot2, w.Nq, w.Nkv)
        kms = [float(np.mean([x[a].elapsed_time(x[a + 1]) for x in ev2])) for a in range(3)]
        tt = {"ms": round(float(np.mean([x[0].elapsed_time(x[3]) for x in ev2])), 4),
              "kernels_ms": {"quantize": round(kms[0], 4), "pass1": round(kms[1], 4),
                             "pass2": round(kms[2], 4)},
              "hot_cells": round(h2 / max(c2, 1), 5)}
        if ref is not None:
            o2 = b2.out.float()
            cos2 = torch.nn.functional.cosine_similarity(o2.reshape(-1, w.D),
                                                         ref.reshape(-1, w.D), dim=1)
            tt["vs_exact"] = {"cos_min": round(float(cos2.min()), 6),
                              "cos_median": round(float(cos2.median()), 6),
                              "max_abs": round(float((o2 - ref).abs().max()), 5)}
        del b2
        return tt

    def prob(**kw):
        return apa.problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D,
                           dtype=apa.APA_F16 if w.dtype == "fp16" else apa.APA_BF16,
                           scale=w.scale, **kw)

    ef_or_none = ef if "apa_vs_exact" in res else None
    if not args.no_variants and w.D <= 256:
        # the pages' second-hunt accuracy fixes: Q plus its FP4 residual term,
        # K block exponents by least squared error, and both
        for name, qt, kl in (("two_term_q", 2, 0), ("k_lsq", 1, 1), ("two_term_q_k_lsq", 2, 1)):
            res[name] = variant(prob(q_terms=qt, k_lsq=kl), ref=ef_or_none)
            print("[bench] %s %.3f ms" % (name, res[name]["ms"]), file=sys.stderr, flush=True)

    if not args.no_variants:
        # the value-norm weighted hot test: on these inputs, and on the same
        # inputs with outlier values (64 tiles per KV head whose values are 8x
        # the rest's), the mass test and the weighted test against the exact
        # output of those inputs
        vw = {"inputs": variant(prob(hot_weight=1), ref=ef_or_none)}
        Vo = V_host.copy()
        outlier_value_tiles(Vo, 64, 8.0, seed=5, dtype=w.dtype)
        vo = torch.from_numpy(Vo).to(dt).cuda()
        del Vo
        eo2 = torch.empty_like(q)
        apa.exact(p, q, k, vo, eo2, None, stream=stream)
        ref2 = eo2.float()
        del eo2
        vw["outlier_values"] = {
            "recipe": "64 tiles per KV head keep their values, all other keys' values / 8",
            "mass_test": variant(prob(), vv=vo, ref=ref2),
            "weighted_test": variant(prob(hot_weight=1), vv=vo, ref=ref2)}
        del vo, ref2
        res["value_norm_weight"] = vw
        print("[bench] value-norm weight %.3f ms" % vw["inputs"]["ms"], file=sys.stderr,
              flush=True)

    if w.eps_sweep and not args.no_sweep:
        # each eps: the same step, warmed up (20 steps: after the all-exact
        # launches the clocks take several steps to settle again), with its
        # kernels timed apart over 20 steps
        sweep = {}
        for e2 in w.eps_sweep:
            for _ in range(20):
                step_eps(apa, p, q, k, v, bufs, e2, stream, None)
            torch.cuda.synchronize()
            evs = []
            t0 = time.perf_counter()
            for _ in range(20):
                step_eps(apa, p, q, k, v, bufs, e2, stream, evs)
            torch.cuda.synchronize()
            ms2 = (time.perf_counter() - t0) * 1e3 / 20
            kms = [float(np.mean([x[a].elapsed_time(x[a + 1]) for x in evs])) for a in range(3)]
            hot2 = apa_hot_mask(p, bufs.bits)
            c2, h2, vp2, hp2 = cell_counts(hot2, w.Nq, w.Nkv)
            sweep[str(e2)] = {"ms": round(ms2, 4), "hot_cells": round(h2 / max(c2, 1), 5),
                              "kernels_ms": {"quantize": round(kms[0], 4),
                                             "pass1": round(kms[1], 4),
                                             "pass2": round(kms[2], 4)}}
            if "exact" in res:
                sweep[str(e2)]["apa_speedup_vs_exact"] = round(res["exact"]["ms"] / ms2, 3)
        res["eps_sweep"] = sweep

    if not args.no_window and w.causal:
        # the page's sliding-window case: each row sees its 4096 most recent
        # keys; APA (same eps) and the all-exact path on the same inputs
        W = 4096
        pw = apa.problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D,
                         dtype=apa.APA_F16 if w.dtype == "fp16" else apa.APA_BF16,
                         scale=w.scale, window=W)
        bw = apa.alloc(pw)
        evw = []
        for i in range(5 + 20):
            step_eps(apa, pw, q, k, v, bw, eps, stream, evw if i >= 5 else None)
        torch.cuda.synchronize()
        kms = [float(np.mean([x[a].elapsed_time(x[a + 1]) for x in evw])) for a in range(3)]
        tot = float(np.mean([x[0].elapsed_time(x[3]) for x in evw]))
        eow = torch.empty_like(q)
        for _ in range(5):
            apa.exact(pw, q, k, v, eow, None, stream=stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10):
            apa.exact(pw, q, k, v, eow, None, stream=stream)
        torch.cuda.synchronize()
        ewms = (time.perf_counter() - t0) * 1e3 / 10
        cosw = torch.nn.functional.cosine_similarity(bw.out.float().reshape(-1, w.D),
                                                     eow.float().reshape(-1, w.D), dim=1)
        hotw = apa_hot_mask(pw, bw.bits)
        res["sliding_window"] = {
            "window": W, "ms": round(tot, 4),
            "kernels_ms": {"quantize": round(kms[0], 4), "pass1": round(kms[1], 4),
                           "pass2": round(kms[2], 4)},
            "exact_ms": round(ewms, 4), "causal_ms": round(ms, 4),
            "hot_groups_tiles": int(hotw.sum()),
            "apa_vs_exact_cos_min": round(float(cosw.min()), 6),
            "page_ms_window_vs_causal": [0.804, 6.053]}
        del bw
        print("[bench] window %d: %.3f ms (exact %.3f)" % (W, tot, ewms), file=sys.stderr,
              flush=True)

    if not args.no_ring and w.D <= 256:
        # the page's KV window ring: the FP4 K/V copy held to a sink tile plus
        # two halves of 96 tiles per KV head, segments coded on a second
        # stream while pass 1 walks the previous one; the same step otherwise
        R = 96
        pr = apa.problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D,
                         dtype=apa.APA_F16 if w.dtype == "fp16" else apa.APA_BF16,
                         scale=w.scale, ring_tiles=R)
        br = apa.alloc(pr)
        evr = []
        for i in range(10 + 20):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            apa.ring_pass1(pr, q, k, v, br.fp4, eps, br.cold_m, br.cold_l, br.cold_o, br.bits,
                           None, ws=br.ws_ring, stream=stream)
            e[1].record(stream)
            apa.pass2(pr, q, k, v, br.fp4, br.bits, br.cold_m, br.cold_l, br.cold_o, True,
                      out=br.out, lse=br.lse, ws=br.ws_p2, stream=stream)
            e[2].record(stream)
            if i >= 10:
                evr.append(e)
        torch.cuda.synchronize()
        cos_r = torch.nn.functional.cosine_similarity(br.out.float().reshape(-1, w.D),
                                                      out.reshape(-1, w.D), dim=1)
        res["kv_window_ring"] = {
            "ring_tiles": R,
            "ms": round(float(np.mean([x[0].elapsed_time(x[2]) for x in evr])), 4),
            "kernels_ms": {"quantize+pass1": round(float(np.mean([x[0].elapsed_time(x[1])
                                                                  for x in evr])), 4),
                           "pass2": round(float(np.mean([x[1].elapsed_time(x[2]) for x in evr])),
                                          4)},
            "fp4_bytes": apa.fp4_bytes(pr), "fp4_bytes_without_ring": apa.fp4_bytes(p),
            "page_fp4_mib": 13.6,
            "vs_main_output_cos_min": round(float(cos_r.min()), 6)}
        del br
        print("[bench] ring %d: %.3f ms" % (R, res["kv_window_ring"]["ms"]), file=sys.stderr,
              flush=True)

    if not args.no_fused and apa.workspace_bytes(p, apa.CALL_FUSED) > 0:
        # both passes in one persistent launch (f1), interleaved step by step
        # with the separate launches on the same inputs so both see the same
        # clocks; its output must equal theirs bit for bit
        bf = apa.alloc(p, with_fused=True)
        evf, evs = [], []
        for i in range(20 + 20):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            apa.quantize(p, q, k, v, bf.fp4, bf.ws_q, stream)
            e[1].record(stream)
            apa.fused(p, q, k, v, bf.fp4, eps, bf.cold_m, bf.cold_l, bf.cold_o, bf.bits, bf.out,
                      lse=bf.lse, ws=bf.ws_fused, stream=stream)
            e[2].record(stream)
            s3 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            s3[0].record(stream)
            step(False)
            s3[1].record(stream)
            if i >= 20:
                evf.append(e)
                evs.append(s3)
        torch.cuda.synchronize()
        L = apa.fp4_layout(p)
        st_word = int(bf.fp4[L.status:L.status + 4].cpu().numpy().view(np.uint32)[0])
        fms = float(np.mean([x[0].elapsed_time(x[2]) for x in evf]))
        sms = float(np.mean([x[0].elapsed_time(x[1]) for x in evs]))
        res["single_launch"] = {
            "ms": round(fms, 4),
            "kernels_ms": {"quantize": round(float(np.mean([x[0].elapsed_time(x[1])
                                                             for x in evf])), 4),
                           "pass1+pass2 (one launch)": round(float(np.mean(
                               [x[1].elapsed_time(x[2]) for x in evf])), 4)},
            "separate_launches_ms": round(sms, 4),
            "tflops": round(flop / (fms * 1e-3) / 1e12, 3),
            "output_equal_to_separate": bool(torch.equal(bf.out, bufs.out) and
                                             torch.equal(bf.lse, bufs.lse)),
            "wait_gave_up": bool(st_word & 2)}
        del bf
        print("[bench] single launch %.3f ms (separate %.3f)" % (fms, sms), file=sys.stderr,
              flush=True)

    if not args.no_cpu:
        # one worker thread per core of the host share a GPU gets (16 here,
        # whatever the host's visible core count)
        threads = max(1, min(16, os.cpu_count() or 1))
        print("[bench] cpu baseline (%d groups, %d threads)" % (args.cpu_groups, threads),
              file=sys.stderr, flush=True)
        res["cpu_baseline"], res["vs_fp64"] = cpu_legs(w, eps, args.cpu_groups, threads,
                                                        gpu_out_host, gpu_hot_host,
                                                        exact_out_host)

    print(json.dumps(res), flush=True)


def step_eps(apa, p, q, k, v, bufs, eps, stream, evs):
    import torch
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if evs is not None else None
    if e:
        e[0].record(stream)
    apa.quantize(p, q, k, v, bufs.fp4, bufs.ws_q, stream)
    if e:
        e[1].record(stream)
    apa.pass1(p, bufs.fp4, eps, bufs.cold_m, bufs.cold_l, bufs.cold_o, bufs.bits, None,
              ws=bufs.ws_p1, stream=stream)
    if e:
        e[2].record(stream)
    apa.pass2(p, q, k, v, bufs.fp4, bufs.bits, bufs.cold_m, bufs.cold_l, bufs.cold_o, True,
              out=bufs.out, lse=bufs.lse, ws=bufs.ws_p2, stream=stream)
    if e:
        e[3].record(stream)
        evs.append(e)


def apa_hot_mask(p, bits):
    import torch
    torch.cuda.synchronize()
    NT = -(-p.Nkv // 64)
    NG = -(-p.Nq // 16)
    W = -(-NT // 32)
    wv = bits.cpu().numpy().view(np.uint32)[:p.B * p.Hq * NG * W].reshape(p.B, p.Hq, NG, W)
    b = (wv[..., None] >> np.arange(32, dtype=np.uint32)) & 1
    return b.reshape(p.B, p.Hq, NG, W * 32)[..., :NT].astype(bool)


if __name__ == "__main__":
    main()
