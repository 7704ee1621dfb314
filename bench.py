"""Benchmark: one step = the whole hot path on one batch of synthetic input.

Step = compress (probe scores, propagation, slots, prototype trees, floor +
auction, pack) + T_dec decode steps over the full cache and over the
compressed cache + per-step KL through the vocab projection. Inputs are
generated on the GPU and resident in HBM before timing starts. The default
workload is the ragged batch: 16 sequences of 2K-32K tokens, 32 layers x 8 KV
heads, 25% budget, 256 decode steps.

Prints ONE JSON line. `value` is KV tokens compressed per second, T / t_compress
(t_compress: HIP events on the library's stream around the compression calls,
median over the timed steps); whole-step throughput (T / step time) is
reported beside it. The decode figures are algorithmic bytes (every packed K/V
byte and ln mu, the appended tokens, the queries, each once) per decode call
divided by the median event time of the calls over each cache; `roofline`
is the call over the 25% cache.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="ragged")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-variants", action="store_true",
                    help="measure only the variants (one JSON object with a 'variants' key); for profiling")
    ap.add_argument("--variants", action="store_true",
                    help="also measure the selection variants beside the headline line (head-level hybrid, "
                         "tree splits, slots from three depths, step-wise eviction, dense and A r propagation)")
    ap.add_argument("--variant", action="append", default=None, metavar="NAME",
                    help="with --variants/--only-variants: measure only these (head_hybrid_0.2, tree_splits, "
                         "dp_3depths_surprisal, stepwise, dense_rollout, ar_direction); repeatable")
    ap.add_argument("--trace-summary", default=None, metavar="CSV",
                    help="only summarize a rocprofv3 kernel_trace.csv of a bench run (per kernel, the decode "
                         "kernels split by cache: the compressed cache's calls launch fewer workgroups), then exit")
    ap.add_argument("--trace-steps", type=int, default=0, metavar="N",
                    help="with --trace-summary: the bench steps the trace covers (warm-up included), to split "
                         "kernels launched a few times a step by launch position")
    ap.add_argument("--counter-summary", default=None, metavar="CSV",
                    help="only summarize a rocprofv3 --pmc counter_collection.csv of a bench run (mean counter "
                         "value per dispatch of each kernel, the decode kernels split by cache), then exit")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring this GPU's own HBM read and bf16 MFMA ceilings (kvc_peak_read, "
                         "kvc_peak_mfma) before the timed steps")
    ap.add_argument("--traffic-json", default=None,
                    help="HBM counter record of the decode call (default profiles/decode_<config>_traffic.json)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run five plain device-to-device copies of MIB MiB (to scale HBM byte "
                         "counters against a kernel of known traffic), then exit")
    return ap.parse_args()


def copy_calibration(mib):
    """Five torch copies of `mib` MiB: each reads and writes exactly mib MiB."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "copies": 5}), flush=True)


def measured_traffic(path, name):
    """HBM bytes per decode call from the committed counter summary, or None
    when it covers another workload or the decode source changed since."""
    import hashlib
    try:
        tj = json.load(open(path))
        src = os.path.join(ROOT, "eviction_probe_softmax_amd", "csrc", "decode.hip")
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except (OSError, ValueError):
        return None
    if tj.get("config") != name or tj.get("decode_source_sha256_16") != sha:
        return None
    return tj.get("traffic_bytes_per_call")


def describe(cfg):
    lens = cfg.lens if len(cfg.lens) <= 4 else f"{len(cfg.lens)} ragged, sum {sum(cfg.lens)}"
    slots = "token-level top-B" if cfg.token_mode else (
        f"DP slots {cfg.slot_min}-{cfg.slot_max}" if cfg.slot_len == 0 else f"fixed {cfg.slot_len}-token slots")
    return (f"{cfg.name}: S={cfg.S} L={lens} Ly={cfg.Ly} H={cfg.H} G={cfg.G} d={cfg.d} {cfg.dtype}, "
            f"{slots}, budget {cfg.budget_ratio:g}, {cfg.T_dec} decode steps, vocab {cfg.vocab}")


def cpu_baseline(cfg, inp):
    """The C++ oracle (fp64, OpenMP over units) timed on this host's cores on
    a bounded part of the same inputs: the first whole sequences of the batch
    up to about 40% of its tokens (the whole job for a single sequence).
    Budgets are per sequence and nothing in the path crosses sequences, so
    this is a complete sub-job, not an extrapolation: value = its tokens / its
    compression time. One decode step over its packed cache is timed too."""
    import numpy as np
    import torch
    from oracle import cpp_oracle as co
    cu = [int(x) for x in inp["cu_seqlens"]]
    k = 1
    while k < cfg.S and cu[k] < 0.4 * cfg.T:
        k += 1
    n_tok = cu[k]
    sub = {"cu_seqlens": torch.tensor(cu[:k + 1], dtype=torch.int64),
           "K": inp["K"][:, :, :n_tok].cpu(), "V": inp["V"][:, :, :n_tok].cpu(), "Qp": inp["Qp"][:k].cpu(),
           "Qctx": inp["Qctx"][:, :, :n_tok].cpu(), "Qd": inp["Qd"][:, :k].cpu(), "Kd": inp["Kd"][:, :, :k].cpu(),
           "Vd": inp["Vd"][:, :, :k].cpu(), "W": inp["W"].cpu(), "hidden": None, "surprisal": None}
    if inp.get("hidden") is not None:
        h = inp["hidden"]
        sub["hidden"] = (h[:, :n_tok] if h.dim() == 3 else h[:n_tok]).cpu()
    sc = cfg.replace(S=k, lens=list(cfg.lens[:k]))
    timings = {}
    t0 = time.perf_counter()
    out = co.compress(sub, sc, timings=timings)
    t_comp = time.perf_counter() - t0
    t = cfg.T_dec - 1
    t1 = time.perf_counter()
    co.decode_step(out["cache"], sub["Kd"], sub["Vd"], sub["Qd"][t], t, cfg.G)
    t_dec = time.perf_counter() - t1
    elt = inp["K"].element_size()
    n_comp = int(np.asarray(out["cache"]["seg_len"], dtype=np.int64).sum())
    dec_bytes = n_comp * (2 * cfg.d * elt + 4) + k * cfg.Ly * cfg.H * (t + 1) * 2 * cfg.d * elt
    threads = co.threads()
    return {"value": round(n_tok / t_comp, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"C++ oracle (fp64, OpenMP, {threads} threads) compressing the first {k} of {cfg.S} "
                       f"sequences of the same inputs ({n_tok} of {cfg.T} tokens, whole sequences) in "
                       f"{t_comp:.1f} s, measured; stages " +
                       ", ".join(f"{kk} {v:.1f} s" for kk, v in timings.items())),
            "decode_gbps_25pct": round(dec_bytes / t_dec / 1e9, 2)}


def measure_variants(cfg, inp, full, x_full, kl_op, stream, steps=2, names=None):
    """Selection variants on the same inputs, outside the headline value:
    compression time, packed entries, decode time per call over the packed
    cache and the per-step KL against the full cache (x_full of the timed
    steps). Head-level hybrid: 20% of the (layer, KV head) units kept whole
    (DistillCache paper, Appendix E.3). Tree splits: curvature-candidate cuts
    (DP slots only) and salient three-way splits (GraceKV page, technical
    details). Step-wise eviction: the scoring-MLP
    loop of DistillCache's Algorithm 1 at the same budget ratio. Dense
    rollout: both propagation hops with every token a seed; the "A r"
    direction: both hops with every token a receiver. Slots cut from three
    sampled depths with the surprisal bonus."""
    import numpy as np
    import torch
    from eviction_probe_softmax_amd import kvc
    from eviction_probe_softmax_amd.pipeline import Compressor, _row_view
    out = {}
    S, Td, Dm = cfg.S, cfg.T_dec, cfg.d_model
    want = (lambda n: True) if not names else (lambda n: n in names)  # noqa: E731
    for name, kw in (("head_hybrid_0.2", {"hybrid_frac": 0.2}), ("tree_splits", {"split_mode": 1})):
        if not want(name):
            continue
        vcfg = cfg.replace(**kw)
        comp = Compressor(vcfg, inp["cu_seqlens"], inp["K"].dtype)
        x_comp = torch.empty((S, Td, Dm), dtype=torch.float32, device="cuda")
        comp.compress(inp)  # warm-up
        cms, dms = [], []
        for _ in range(steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            res = comp.compress(inp)
            e[1].record(stream)
            dec = kvc.Decoder(res["cache"], vcfg.G, Td)
            for t in range(Td):
                dec.step(inp["Kd"], inp["Vd"], t + 1, inp["Qd"][t], _row_view(x_comp, t), Td * Dm)
            e[2].record(stream)
            torch.cuda.synchronize()
            cms.append(e[0].elapsed_time(e[1]))
            dms.append(e[1].elapsed_time(e[2]) / Td)
        klv = kl_op(x_full.reshape(S * Td, Dm), x_comp.reshape(S * Td, Dm), inp["W"]).float().cpu().numpy()
        out[name] = {"compress_ms": round(float(np.mean(cms)), 3),
                     "decode_ms_per_call": round(float(np.mean(dms)), 4),
                     "packed_entries": int(res["cache"]["seg_len"].to(torch.int64).sum()),
                     "mean_kl": round(float(klv.mean()), 5), "max_kl": round(float(klv.max()), 5)}
        if vcfg.hybrid_frac > 0:
            out[name]["units_kept_whole"] = int(kvc.hybrid_units(comp.pb, res["head_sens"]).sum())
        if vcfg.split_mode:
            cost = res["trees"]["op_cost"]
            three = cost == 2
            out[name]["three_way_splits"] = int(three.sum())
            out[name]["three_way_taken"] = int((three & (res["taken"] > 0)).sum())
            out[name]["curvature_cuts"] = vcfg.slot_len == 0
    # Slots cut from three sampled depths with the surprisal bonus (DP slots)
    if want("dp_3depths_surprisal") and cfg.slot_len == 0:
        from workload import make_inputs
        vcfg = cfg.replace(n_depth=3, surprisal=True)
        vin = make_inputs(vcfg, device="cuda")
        comp = Compressor(vcfg, vin["cu_seqlens"], vin["K"].dtype)
        comp.compress(vin)  # warm-up
        e3 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e3[0].record(stream)
        res3 = comp.compress(vin)
        e3[1].record(stream)
        torch.cuda.synchronize()
        out["dp_3depths_surprisal"] = {"compress_ms": round(e3[0].elapsed_time(e3[1]), 3),
                                       "slots": int(res3["n_slots"].sum())}
        del vin, comp, res3
    if not (want("stepwise") or want("dense_rollout") or want("ar_direction")):
        return out
    # Step-wise eviction (DistillCache Algorithm 1) with a seeded scoring MLP:
    # one prefill prune, then per decode step append + decode + score + prune
    if want("stepwise"):
        from workload import make_policy
        from eviction_probe_softmax_amd.pipeline import run_stepwise
        pol = make_policy(device="cuda")
        run_stepwise(cfg, inp, pol)  # warm-up
        rec = []
        torch.cuda.synchronize()
        res = run_stepwise(cfg, inp, pol, record=rec)
        torch.cuda.synchronize()
        init_ms = [r[1].elapsed_time(r[2]) for r in rec if r[0] == "init"]
        dec_ms = [r[1].elapsed_time(r[2]) for r in rec if r[0] == "step"]
        prune_ms = [r[2].elapsed_time(r[3]) for r in rec if r[0] == "step"]
        klv = res["kl"].float().cpu().numpy()
        out["stepwise_r%g" % cfg.budget_ratio] = {
            "init_prune_ms": round(float(np.mean(init_ms)), 3),
            "append_decode_ms_per_step": round(float(np.mean(dec_ms)), 4),
            "score_prune_ms_per_step": round(float(np.mean(prune_ms)), 4),
            "cached_entries_last_step": int(sum(res["stepwise"].lengths)) * cfg.Ly * cfg.H,
            "mean_kl": round(float(klv.mean()), 5), "max_kl": round(float(klv.max()), 5)}
    if not (want("dense_rollout") or want("ar_direction")):
        return out
    # Dense rollout: every token a seed in both hops (a causal L x L pass per
    # hop); flops count each causal logit once per pass (rowstats, colsum)
    comp = Compressor(cfg, inp["cu_seqlens"], inp["K"].dtype)
    sc = kvc.score(comp.pb, inp["K"], inp["V"], inp["Qp"])
    causal = sum(L * (L + 1) // 2 for L in cfg.lens)
    flops = cfg.n_hops * 2 * cfg.Ly * cfg.H * cfg.G * causal * 2 * cfg.d
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    if want("dense_rollout"):
        kvc.propagate_dense(comp.pb, inp["K"], inp["Qctx"], sc["r0"])  # warm-up
        e[0].record(stream)
        kvc.propagate_dense(comp.pb, inp["K"], inp["Qctx"], sc["r0"])
        e[1].record(stream)
        torch.cuda.synchronize()
        dms = e[0].elapsed_time(e[1])
        out["dense_rollout"] = {"ms": round(dms, 3), "tflops": round(flops / (dms * 1e-3) / 1e12, 1),
                                "mfma_bf16_frac": round(flops / (dms * 1e-3) / 2.5e15, 4)}
    # the "A r" direction: one causal row pass per hop
    if want("ar_direction"):
        kvc.propagate_ar(comp.pb, inp["K"], inp["Qctx"], sc["r0"])  # warm-up
        e[0].record(stream)
        kvc.propagate_ar(comp.pb, inp["K"], inp["Qctx"], sc["r0"])
        e[1].record(stream)
        torch.cuda.synchronize()
        ams = e[0].elapsed_time(e[1])
        out["ar_direction"] = {"ms": round(ams, 3), "tflops": round(flops / 2 / (ams * 1e-3) / 1e12, 1),
                               "mfma_bf16_frac": round(flops / 2 / (ams * 1e-3) / 2.5e15, 4)}
    return out


def trace_summary(path, nsteps=0):
    """Per-kernel summary of a rocprofv3 kernel_trace.csv (one row a
    dispatch): calls, total and mean microseconds, mean grid. The decode
    kernels are split by cache: within one run the calls over the compressed
    cache launch fewer workgroups than those over the full cache, so the
    dispatches of each decode kernel fall into two grid sizes (per step; the
    tail pieces grow with the step), and the smaller half is the compressed
    cache's. With nsteps (the bench steps the trace covers, warm-up
    included), a kernel launched 2-4 times a step is split by its launch
    position within the step (#1, #2, ...: the probe pass, then the
    propagation hops). Prints a markdown table."""
    import csv
    from collections import defaultdict
    rows = list(csv.DictReader(open(path)))
    key_start = "Start_Timestamp" if "Start_Timestamp" in rows[0] else "Start_Time"
    key_end = "End_Timestamp" if "End_Timestamp" in rows[0] else "End_Time"
    by = defaultdict(list)
    for r in rows:
        name = r["Kernel_Name"]
        dur = (int(r[key_end]) - int(r[key_start])) / 1e3
        grid = int(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0)
        by[name].append((int(r[key_start]), dur, grid))
    out = defaultdict(list)
    for name, lst in by.items():
        short = name.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0].strip()
        if short.split("<")[0] in ("decode_mfma_kernel", "decode_partial_kernel", "decode_merge_kernel",
                                   "decode_layersum_kernel"):
            lst.sort()
            # calls come in (full, compressed) pairs in every decode step
            full, comp = lst[0::2], lst[1::2]
            if comp and sum(g for _, _, g in comp) > sum(g for _, _, g in full):
                full, comp = comp, full
            out[short + " [full cache]"] += full
            out[short + " [25% cache]"] += comp
        elif nsteps and len(lst) % nsteps == 0 and 2 <= len(lst) // nsteps <= 4:
            per = len(lst) // nsteps
            lst.sort()
            for k in range(per):
                out[f"{short} #{k + 1}"] += lst[k::per]
        else:
            out[short or name] += lst
    tot = sum(d for lst in by.values() for _, d, _ in lst)
    print("| kernel | calls | total ms | mean us | median us | mean grid | % of kernel time |")
    print("|---|---|---|---|---|---|---|")
    for name, lst in sorted(out.items(), key=lambda kv: -sum(d for _, d, _ in kv[1])):
        ds = sorted(d for _, d, _ in lst)
        t = sum(ds)
        med = ds[len(ds) // 2]
        print(f"| {name} | {len(ds)} | {t / 1e3:.3f} | {t / len(ds):.2f} | {med:.2f} | "
              f"{sum(g for _, _, g in lst) / len(lst):.0f} | {100 * t / tot:.1f} |")


def counter_summary(path):
    """Mean counter value per dispatch of each kernel in a rocprofv3 --pmc
    counter_collection.csv, the decode kernels split by cache as in
    trace_summary (dispatch order alternates full, compressed). Prints a
    markdown table."""
    import csv
    from collections import defaultdict
    rows = list(csv.DictReader(open(path)))
    disp = {}
    for r in rows:
        key = int(r.get("Dispatch_Id", r.get("Correlation_Id", 0)))
        d = disp.setdefault(key, {"name": r["Kernel_Name"], "grid": int(r.get("Grid_Size", 0) or 0), "c": {}})
        d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    by = defaultdict(list)
    for key in sorted(disp):
        d = disp[key]
        short = d["name"].replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0].strip()
        by[short].append(d)
    out = defaultdict(list)
    for short, lst in by.items():
        if short.split("<")[0] in ("decode_mfma_kernel", "decode_partial_kernel", "decode_merge_kernel",
                                   "decode_layersum_kernel"):
            full, comp = lst[0::2], lst[1::2]
            if comp and sum(x["grid"] for x in comp) > sum(x["grid"] for x in full):
                full, comp = comp, full
            out[short + " [full cache]"] += full
            out[short + " [25% cache]"] += comp
        else:
            out[short] += lst
    names = sorted({c for lst in out.values() for d in lst for c in d["c"]})
    print("| kernel | dispatches | " + " | ".join(f"{c} (mean)" for c in names) + " |")
    print("|---|---|" + "---|" * len(names))
    for short, lst in sorted(out.items()):
        means = [sum(d["c"].get(c, 0.0) for d in lst) / len(lst) for c in names]
        print(f"| {short} | {len(lst)} | " + " | ".join(f"{m:.1f}" for m in means) + " |")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    if args.trace_summary:
        trace_summary(args.trace_summary, args.trace_steps)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import numpy as np
    import torch
    from workload import get_config, make_inputs
    from eviction_probe_softmax_amd import kvc
    from eviction_probe_softmax_amd.pipeline import Compressor, _row_view

    cfg = get_config(args.config)
    dev = "cuda"
    peaks = None
    if not args.no_peaks:
        # the machine's own ceilings, measured before anything else is resident
        peaks = {"hbm_read_gbs": round(kvc.peak_read_gbs(), 1), "mfma_bf16_tflops": round(kvc.peak_mfma_tflops(), 1),
                 "exp_mix_gelems": round(kvc.peak_exp_gelems(), 1),
                 "how": "kvc_peak_read: 2 GiB of nontemporal 16-byte loads, each workgroup streaming one "
                        "contiguous span; kvc_peak_mfma: register-only 32x32x16 bf16 MFMA chains on every SIMD; "
                        "kvc_peak_exp: register-only chains of one v_exp_f32 and three VALU operations (the "
                        "probe passes' per-logit mix), elements per second"}
        print(f"[bench] measured peaks {peaks['hbm_read_gbs']} GB/s, {peaks['mfma_bf16_tflops']} TFLOP/s",
              file=sys.stderr, flush=True)
    t_gen = time.perf_counter()
    inp = make_inputs(cfg, device=dev, seed=args.seed)
    torch.cuda.synchronize()
    print(f"[bench] inputs for {cfg.name} ready in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)
    comp = Compressor(cfg, inp["cu_seqlens"], inp["K"].dtype, device=dev)
    full = kvc.full_view(comp.pb, inp["K"], inp["V"])
    S, Td, Dm = cfg.S, cfg.T_dec, cfg.d_model
    x_full = torch.empty((S, Td, Dm), dtype=torch.float32, device=dev)
    x_comp = torch.empty((S, Td, Dm), dtype=torch.float32, device=dev)
    kl_op = kvc.KL(S * Td, Dm, cfg.vocab, inp["W"].dtype, device=dev)
    if args.only_variants:
        dfull = kvc.Decoder(full, cfg.G, Td)
        for t in range(Td):
            dfull.step(inp["Kd"], inp["Vd"], t + 1, inp["Qd"][t], _row_view(x_full, t), Td * Dm)
        v = measure_variants(cfg, inp, full, x_full, kl_op, torch.cuda.current_stream(), names=args.variant)
        print(json.dumps({"config": {"workload": describe(cfg)}, "variants": v}), flush=True)
        return
    elt = inp["K"].element_size()
    d = cfg.d
    stream = torch.cuda.current_stream()

    def step(record=None):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record is not None else None
        if ev:
            ev[0].record(stream)
        out = comp.compress(inp)
        if ev:
            ev[1].record(stream)
        cache = out["cache"]
        dfull = kvc.Decoder(full, cfg.G, Td)
        dcomp = kvc.Decoder(cache, cfg.G, Td)
        dec_ev = []
        for t in range(Td):
            q = inp["Qd"][t]
            if record is not None:
                e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                e0.record(stream)
            # outputs land directly in x[s, t] (row stride T_dec * d_model)
            dfull.step(inp["Kd"], inp["Vd"], t + 1, q, _row_view(x_full, t), Td * Dm)
            if record is not None:
                e1.record(stream)
            dcomp.step(inp["Kd"], inp["Vd"], t + 1, q, _row_view(x_comp, t), Td * Dm)
            if record is not None:
                e2.record(stream)
                dec_ev.append((e0, e1, e2))
        if ev:
            ev[2].record(stream)
        klv = kl_op(x_full.reshape(S * Td, Dm), x_comp.reshape(S * Td, Dm), inp["W"])
        if ev:
            ev[3].record(stream)
        if record is not None:
            record.append((ev, dec_ev, out, klv))
        return out, klv

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    comp_ms, dec_ms, kl_ms, dfull_ms, dcomp_ms = [], [], [], [], []
    for ev, dec_ev, out, klv in recs:
        comp_ms.append(ev[0].elapsed_time(ev[1]))
        dec_ms.append(ev[1].elapsed_time(ev[2]))
        kl_ms.append(ev[2].elapsed_time(ev[3]))
        for e0, e1, e2 in dec_ev:
            dfull_ms.append(e0.elapsed_time(e1))
            dcomp_ms.append(e1.elapsed_time(e2))
    out, klv = recs[-1][2], recs[-1][3]
    seg_len = out["cache"]["seg_len"].to(torch.int64)
    n_comp = int(seg_len.sum())
    n_full = cfg.T * cfg.Ly * cfg.H
    units = cfg.S * cfg.Ly * cfg.H
    # algorithmic bytes of one decode call: packed K+V (+ ln mu) once, the
    # appended tail (mean over steps) once, the queries once
    tail_mean = (Td + 1) / 2.0
    q_bytes = units * cfg.G * d * elt
    bytes_comp = n_comp * (2 * d * elt + 4) + units * tail_mean * 2 * d * elt + q_bytes
    bytes_full = n_full * 2 * d * elt + units * tail_mean * 2 * d * elt + q_bytes
    med_comp_ms = float(np.median(dcomp_ms))
    med_full_ms = float(np.median(dfull_ms))
    gbs_comp = bytes_comp / (med_comp_ms * 1e-3) / 1e9
    gbs_full = bytes_full / (med_full_ms * 1e-3) / 1e9
    t_compress = float(np.median(comp_ms))
    tpath = args.traffic_json or os.path.join(ROOT, "profiles", f"decode_{cfg.name}_traffic.json")
    traffic = measured_traffic(tpath, cfg.name)
    klh = klv.detach().float().cpu().numpy()
    B, A, F = comp.pb.budgets()
    res = {
        "metric": "KV tokens compressed/sec + decode-attn HBM GB/s at 25% budget; mean KL",
        "value": round(cfg.T / (t_compress / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": describe(cfg), "seq_lens": cfg.lens,
                   "budget_ratio": cfg.budget_ratio, "entries_budget": B, "decode_steps": Td,
                   "vocab": cfg.vocab},
        "compress_ms": round(t_compress, 3),
        "compress_entries_per_s": round(n_full / (t_compress / 1e3), 1),
        "step_tokens_per_s": round(cfg.T / (ms_per_step / 1e3), 1),
        "decode_ms_per_step": round(float(np.median(dec_ms)), 3),
        "decode_comp_ms_per_call": round(med_comp_ms, 4),
        "decode_full_ms_per_call": round(med_full_ms, 4),
        "decode_hbm_gbps_25pct": round(gbs_comp, 1),
        "decode_hbm_gbps_full": round(gbs_full, 1),
        "packed_entries": n_comp,
        "full_entries": n_full,
        "kl_ms": round(float(np.median(kl_ms)), 3),
        "mean_kl": round(float(klh.mean()), 5),
        "max_kl": round(float(klh.max()), 5),
        "roofline": {"bound": "hbm", "kernel": "decode call over the 25% cache (decode_mfma pieces + "
                                               "decode_merge + decode_layersum)",
                     "achieved": round(gbs_comp, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs_comp / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_call": int(bytes_comp), "ms_per_call": round(med_comp_ms, 4),
                     "full_cache": {"achieved": round(gbs_full, 1), "frac": round(gbs_full / HBM_PEAK_GBS, 4),
                                    "bytes_per_call": int(bytes_full), "ms_per_call": round(med_full_ms, 4)}},
        "measured_peaks": peaks,
    }
    if peaks:
        res["roofline"]["peak_measured"] = peaks["hbm_read_gbs"]
        res["roofline"]["frac_measured"] = round(gbs_comp / peaks["hbm_read_gbs"], 4)
    if args.variants:
        res["variants"] = measure_variants(cfg, inp, full, x_full, kl_op, stream, names=args.variant)
    if not args.no_cpu_baseline:
        print("[bench] timing the C++ oracle on the host cores", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, inp)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
