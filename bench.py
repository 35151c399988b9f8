#!/usr/bin/env python3
"""Throughput of the drafter LM head and speculative verification on one MI355X.

Default workload: the Llama-3.1-8B-shaped drafter head (d = 4096, V = 128256, bf16), one
call over 8 sequences x 6 draft steps = 48 hidden-state rows.  One step is one call of the
SlimSpec low-rank head (r = 512) with fused log-softmax and temperature-1 sampling; `value`
is rows scored per second.  Secondary legs, reported in the same JSON line: the same head at
1 x 6 rows and greedy, the dense V x d head, the SpecVocab head (d' = 256, k = 2048) at this
shape, and batched verification (64 sequences, gamma 5, V = 151936).

Weights are copied to several rotated device buffers whose total exceeds the 256 MB
Infinity Cache, so each timed call streams its weights from HBM.  Per-kernel durations come
from events the library records around each launch on the launch stream (sh_trace_*).

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
METRIC = "draft LM-head tokens/s and % HBM roofline (V=128256,d=4096); verify tokens/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--legs", default="all",
                   help="comma list of legs (lowrank48,lowrank48g,lowrank6,lowrank48logits,lowrank8x6,dense48,"
                        "dense6,specvocab1,specvocab16,specvocabq1,specvocabq16,verify,verifys0.5,verifys2,verifyg,verifysparse,verifytree,"
                        "adaptive48,adaptive48s,trimmed48,trimmed6,trimmedceiling,gptoss192) or 'all' "
                        "or 'headline'")
    p.add_argument("--rotate", type=int, default=5, help="device copies of each weight set")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-trace", action="store_true", help="skip the per-kernel event pass")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a device-to-device copy of this many MiB (counter calibration)")
    p.add_argument("--traffic-summary", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                   help="only write the HBM traffic summary of the headline kernel from four rocprofv3 "
                        "--pmc counter_collection.csv files (head leg FETCH_SIZE, WRITE_SIZE; the "
                        "calibration copy's FETCH_SIZE, WRITE_SIZE)")
    p.add_argument("--pmc-summary", nargs="+", metavar="CSV",
                   help="only print, as a markdown table, the mean per dispatch of every counter in the given "
                        "rocprofv3 --pmc counter_collection.csv files, per kernel")
    return p.parse_args()


def sha_of(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


KERNEL_SOURCES = ["drafter_lm_head_slimspec_amd/csrc/head_tile.hip",
                  "drafter_lm_head_slimspec_amd/csrc/device_common.h"]
HEAD_KERNEL = "k_head_tile"
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic_head_tile_llama_lowrank_M48.json")
COPY_MIB = 1024
LEG_PMC_ARGS = "--steps 5 --warmup 1 --no-trace --no-cpu-baseline --legs lowrank48"
COPY_LAUNCHES = 3


def counter_kib(path, kernel, counter, launches=None):
    """KiB per dispatch of `counter` over the dispatches whose name contains `kernel`; with
    `launches`, the sum over all matching dispatches divided by that many launches (a copy
    the runtime splits into several dispatches)."""
    import csv
    vals = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if kernel in row["Kernel_Name"] and row["Counter_Name"] == counter:
                d = row["Dispatch_Id"]
                vals[d] = vals.get(d, 0.0) + float(row["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel} in {path}")
    tot = sum(vals.values())
    return tot / launches if launches else tot / len(vals), len(vals)


def traffic_summary(paths):
    """HBM bytes per launch of the headline kernel: its FETCH_SIZE / WRITE_SIZE readings, each
    scaled by the ratio of a device copy's known byte count to the same counter's reading."""
    fpath, wpath, cfpath, cwpath = paths
    fk, nf = counter_kib(fpath, HEAD_KERNEL, "FETCH_SIZE")
    wk, nw = counter_kib(wpath, HEAD_KERNEL, "WRITE_SIZE")
    copy_bytes = COPY_MIB << 20
    cf, _ = counter_kib(cfpath, "copyBuffer", "FETCH_SIZE", COPY_LAUNCHES)
    cw, _ = counter_kib(cwpath, "copyBuffer", "WRITE_SIZE", COPY_LAUNCHES)
    fscale, wscale = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    from drafter_lm_head_slimspec_amd import configs
    w = configs.LLAMA
    alg = w.V * w.r * 2 + 48 * w.r * 2
    hbm = fk * 1024 * fscale + wk * 1024 * wscale
    out = {"kernel": HEAD_KERNEL, "workload": "llama3.1-8b-head low-rank r=512, 48 rows, sampling",
           "source_sha256": sha_of(KERNEL_SOURCES), "source_files": KERNEL_SOURCES,
           "dispatches": {"fetch": nf, "write": nw},
           "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk, "copy_calibration_mib": COPY_MIB,
           "fetch_scale": fscale, "write_scale": wscale, "hbm_bytes_per_launch": hbm,
           "alg_bytes_per_launch": alg, "traffic_over_alg": hbm / alg,
           "commands": [
               f"rocprofv3 --pmc {c} --output-format csv -d {os.path.dirname(p)} -o run -- "
               f"python3 bench.py {args}"
               for c, p, args in (("FETCH_SIZE", fpath, LEG_PMC_ARGS), ("WRITE_SIZE", wpath, LEG_PMC_ARGS),
                                  ("FETCH_SIZE", cfpath, f"--copy-calibration {COPY_MIB}"),
                                  ("WRITE_SIZE", cwpath, f"--copy-calibration {COPY_MIB}"))]
           + ["python3 bench.py --traffic-summary " + " ".join(paths)]}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({"hbm_bytes_per_launch": hbm, "traffic_over_alg": hbm / alg}))


def pmc_summary(paths):
    """Mean per dispatch of each counter, per kernel (name up to its argument list), over the
    given rocprofv3 counter_collection.csv files; one markdown row per kernel."""
    import csv
    per = {}   # kernel -> counter -> {dispatch: value}
    for path in paths:
        with open(path) as f:
            for row in csv.DictReader(f):
                kn = row["Kernel_Name"].split("(")[0][:80]
                c = per.setdefault(kn, {}).setdefault(row["Counter_Name"], {})
                key = (path, row["Dispatch_Id"])
                c[key] = c.get(key, 0.0) + float(row["Counter_Value"])
    counters = sorted({c for k in per.values() for c in k})
    print("| kernel | dispatches | " + " | ".join(counters) + " |")
    print("|---|---|" + "---|" * len(counters))
    for kn in sorted(per):
        n = max(len(v) for v in per[kn].values())
        cells = []
        for c in counters:
            v = per[kn].get(c)
            cells.append(f"{sum(v.values()) / len(v):.6g}" if v else "")
        print(f"| `{kn}` | {n} | " + " | ".join(cells) + " |")


def read_bandwidth(sh, torch, dev, reps=10):
    """Attainable HBM read rate: the library's flat read kernel over 1 GiB (four times the
    Infinity Cache, so every read comes from HBM), timed with events around each launch."""
    nbytes = 1 << 30
    buf = torch.arange(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        sh.read_probe(buf, sink)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        sh.read_probe(buf, sink)
    e.record()
    torch.cuda.synchronize()
    us = 1000.0 * s.elapsed_time(e) / reps
    del buf
    return {"GBps": nbytes / (us * 1e-6) / 1e9, "bytes": nbytes, "us_per_read": us,
            "kernel": "k_read_probe: 1024 x 256 threads, flat grid-stride 16-byte loads, 4 in flight per thread",
            "reads": reps}


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(args.traffic_summary)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.gpus != 1:
        log(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for {args.gpus}).")
        sys.exit(2)
    import torch
    from drafter_lm_head_slimspec_amd import configs, spechead as sh, synth

    sh.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(COPY_LAUNCHES):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": COPY_LAUNCHES}))
        return

    w = configs.LLAMA
    d, V, r, dp, k = w.d, w.V, w.r, w.dprime, w.k
    seeds = w.seeds
    legs_all = ["lowrank48", "lowrank48g", "lowrank6", "lowrank48logits", "lowrank8x6", "gptoss192", "adaptive48",
                "adaptive48s", "dense48", "dense6", "trimmed48", "trimmed6", "trimmedceiling",
                "specvocab1", "specvocab16", "specvocabq1", "specvocabq16",
                "verify", "verifys0.5", "verifys2", "verifyg", "verifysparse", "verifytree"]
    if args.legs == "all":
        legs = legs_all
    elif args.legs == "headline":
        legs = ["lowrank48"]
    else:
        legs = [x for x in args.legs.split(",") if x]
    R = max(1, args.rotate)

    def bf(arr):
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)

    t0 = time.time()
    log("generating inputs ...")
    h48_np = synth.hidden(48, d, "bf16", seeds["hidden"])
    h6_np = h48_np[:6].copy()
    Wd_np, Wu_np = synth.lowrank_weights(V, d, r, "bf16", seeds["weights"])
    Wd = [bf(Wd_np)] + []
    Wu = [bf(Wu_np)]
    for _ in range(R - 1):
        Wd.append(Wd[0].clone())
        Wu.append(Wu[0].clone())
    h48 = bf(h48_np)
    h6 = bf(h6_np)
    need_dense = any(x.startswith(("dense", "trimmed")) or x in ("specvocab1", "specvocab16") for x in legs)
    W = bf(synth.dense_weights(V, d, "bf16", seeds["weights"])) if need_dense else None
    log(f"  inputs ready in {time.time() - t0:.1f}s")

    results = {}
    kernel_trace = {}
    line_extra = {}

    def timed(calls, steps, warmup):
        n = len(calls)
        for i in range(warmup):
            calls[i % n]()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(steps):
            calls[i % n]()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / steps

    def traced(calls, steps):
        n = len(calls)
        sh.trace_enable(8 * steps + 64)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(steps):
            calls[i % n]()
        e.record()
        torch.cuda.synchronize()
        tr = sh.trace_read()
        sh.trace_enable(0)
        return s.elapsed_time(e) / steps, tr

    def run_leg(name, calls, rows, alg_bytes, unit_rows="rows"):
        ms = timed(calls, args.steps, args.warmup)
        out = {"ms_per_call": ms, "us_per_call": 1000 * ms, "tokens_per_s": rows / (ms / 1000.0),
               "alg_bytes": alg_bytes, "hbm_frac": alg_bytes / (ms / 1000.0) / (HBM_PEAK_GBS * 1e9),
               "rows": rows, "unit": unit_rows}
        if not args.no_trace:
            ms_t, tr = traced(calls, args.steps)
            out["ms_per_call_traced"] = ms_t
            out["kernels"] = {kname: {"count": v["count"], "avg_us": v["total_us"] / v["count"],
                                      "min_us": v["min_us"], "max_us": v["max_us"]}
                              for kname, v in tr.items()}
            kernel_trace[name] = out["kernels"]
        results[name] = out
        log(f"  {name:12s} {1000 * ms:9.2f} us/call  {out['tokens_per_s']:12.0f} {unit_rows}/s  "
            f"{100 * out['hbm_frac']:5.1f}% of HBM roofline")
        return out

    def lowrank_calls(h, M, mode, logits=False):
        calls = []
        for i in range(R):
            tok = torch.empty(M, dtype=torch.int32, device=dev)
            lse = torch.empty(M, dtype=torch.float32, device=dev)
            lp = torch.empty(M, dtype=torch.float32, device=dev)
            zl = torch.empty(M, V, dtype=torch.float32, device=dev) if logits else None
            need = sh.load().sh_head_workspace_bytes(sh.OP_LOWRANK, M, d, r, V, 0)
            ws = torch.zeros(need, dtype=torch.uint8, device=dev)
            calls.append(sh.prepared("draft_head_lowrank", h, M, d, Wd[i], r, Wu[i], V, sh.SH_BF16,
                                     mode, 1.0, seeds["philox"], i, tok, lse, lp, zl, ws, need,
                                     torch.cuda.current_stream().cuda_stream))
            calls[-1].keep = (tok, lse, lp, zl, ws)
        return calls

    def dense_calls(h, M, mode):
        tok = torch.empty(M, dtype=torch.int32, device=dev)
        lse = torch.empty(M, dtype=torch.float32, device=dev)
        lp = torch.empty(M, dtype=torch.float32, device=dev)
        need = sh.load().sh_head_workspace_bytes(sh.OP_DENSE, M, d, 0, V, 0)
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        c = sh.prepared("draft_head_dense", h, M, d, W, V, sh.SH_BF16, mode, 1.0, seeds["philox"], 0,
                        tok, lse, lp, None, ws, need, torch.cuda.current_stream().cuda_stream)
        c.keep = (tok, lse, lp, ws)
        return [c]

    lowrank_bytes = lambda M: (r * d + V * r + M * d) * 2 + M * 12
    if "lowrank48" in legs:
        run_leg("lowrank48", lowrank_calls(h48, 48, sh.SAMPLE), 48, lowrank_bytes(48))
    if "lowrank48g" in legs:
        run_leg("lowrank48g", lowrank_calls(h48, 48, sh.GREEDY), 48, lowrank_bytes(48))
    if "lowrank6" in legs:
        run_leg("lowrank6", lowrank_calls(h6, 6, sh.SAMPLE), 6, lowrank_bytes(6))
    if "lowrank48logits" in legs:
        # the same call also writing the raw logits [48, V] float32 (their bytes counted)
        o = run_leg("lowrank48logits", lowrank_calls(h48, 48, sh.SAMPLE, logits=True), 48,
                    lowrank_bytes(48) + 48 * V * 4)
        o["config"] = {"logits": "float32 [48, V] written"}
    if "lowrank8x6" in legs:
        # an autoregressive drafter: gamma = 6 calls of B = 8 rows, each on its own hidden
        # states, one step = the 6 calls (every call streams W_up again)
        hs = [bf(synth.hidden(8, d, "bf16", seeds["hidden"] + 300 + t)) for t in range(6)]
        per_t = [lowrank_calls(hs[t], 8, sh.SAMPLE) for t in range(6)]
        steps = []
        for i in range(R):
            seq = [per_t[t][i] for t in range(6)]

            def step(seq=seq):
                for c in seq:
                    c()
            step.keep = seq
            steps.append(step)
        o = run_leg("lowrank8x6", steps, 48, 6 * lowrank_bytes(8))
        o["config"] = {"calls_per_step": 6, "rows_per_call": 8, "note": "gamma calls of B rows"}
    dense_bytes = lambda M: (V * d + M * d) * 2 + M * 12
    if "dense48" in legs:
        run_leg("dense48", dense_calls(h48, 48, sh.SAMPLE), 48, dense_bytes(48))
    if "dense6" in legs:
        run_leg("dense6", dense_calls(h6, 6, sh.SAMPLE), 6, dense_bytes(6))

    def specvocab_legs(prefix, wl, Vs, Uw):
        """SpecVocab at vocabulary size Vs (d, d', k of workload wl), exact rows from Uw [Vs, d]."""
        Wdp_np, Wv_np, _ = synth.specvocab_weights(Vs, wl.d, wl.dprime, "bf16", wl.seeds["weights"], with_U=False)
        Wdp = [bf(Wdp_np)]
        Wv = [bf(Wv_np)]
        for _ in range(R):
            Wdp.append(Wdp[0].clone())
            Wv.append(Wv[0].clone())
        for M in (1, 16):
            name = f"{prefix}{M}"
            if name not in legs:
                continue
            calls, union_rows = [], []
            for i in range(R + 1):
                hi = bf(synth.hidden(M, wl.d, "bf16", wl.seeds["hidden"] + 100 + i))
                idx = torch.empty(M, wl.k, dtype=torch.int32, device=dev)
                zl = torch.empty(M, wl.k, dtype=torch.float32, device=dev)
                q = torch.empty(M, wl.k, dtype=torch.float32, device=dev)
                tok = torch.empty(M, dtype=torch.int32, device=dev)
                lse = torch.empty(M, dtype=torch.float32, device=dev)
                lp = torch.empty(M, dtype=torch.float32, device=dev)
                need = sh.load().sh_head_workspace_bytes(sh.OP_SPECVOCAB, M, wl.d, wl.dprime, Vs, wl.k)
                ws = torch.zeros(need, dtype=torch.uint8, device=dev)
                c = sh.prepared("draft_head_specvocab", hi, M, wl.d, Wdp[i], wl.dprime, Wv[i], Uw, Vs, wl.k,
                                sh.SH_BF16, sh.SAMPLE, 1.0, wl.seeds["philox"], i, idx, zl, q, tok, lse, lp, ws,
                                need, torch.cuda.current_stream().cuda_stream)
                c.keep = (hi, idx, zl, q, tok, lse, lp, ws)
                c()
                torch.cuda.synchronize()
                union_rows.append(len(np.unique(idx.cpu().numpy())))
                calls.append(c)
            u = float(np.mean(union_rows))
            alg = (wl.dprime * wl.d + Vs * wl.dprime) * 2 + u * wl.d * 2 + M * wl.d * 2 + M * wl.k * 12
            out = run_leg(name, calls, M, alg)
            out["union_rows"] = u
            out["config"] = {"workload": wl.name if Vs == wl.V else f"specvocab at V={Vs}", "d": wl.d, "V": Vs,
                             "dprime": wl.dprime, "k": wl.k, "rows": M}

    # SpecVocab at the Llama vocabulary (the headline's V = 128256) ...
    if any(x in legs for x in ("specvocab1", "specvocab16")):
        specvocab_legs("specvocab", w, V, W)
    # ... and at the Qwen3-8B shape (V = 151936), its exact rows from a V x d matrix of that size
    if any(x in legs for x in ("specvocabq1", "specvocabq16")):
        qw = configs.QWEN
        WQ = bf(synth.dense_weights(qw.V, qw.d, "bf16", qw.seeds["weights"]))
        specvocab_legs("specvocabq", qw, qw.V, WQ)
        del WQ

    # GPT-OSS-20B-shaped low-rank head: d 2880, V 201088, r 360, 32 sequences x 6 = 192 rows, T 0.7
    if "gptoss192" in legs:
        g = configs.GPTOSS
        Mg = g.Ms[0]
        hg = bf(synth.hidden(Mg, g.d, "bf16", g.seeds["hidden"]))
        gd_np, gu_np = synth.lowrank_weights(g.V, g.d, g.r, "bf16", g.seeds["weights"])
        GWd = [bf(gd_np)]
        GWu = [bf(gu_np)]
        del gd_np, gu_np
        for _ in range(R - 1):
            GWd.append(GWd[0].clone())
            GWu.append(GWu[0].clone())
        calls = []
        for i in range(R):
            tok = torch.empty(Mg, dtype=torch.int32, device=dev)
            lse = torch.empty(Mg, dtype=torch.float32, device=dev)
            lp = torch.empty(Mg, dtype=torch.float32, device=dev)
            need = sh.load().sh_head_workspace_bytes(sh.OP_LOWRANK, Mg, g.d, g.r, g.V, 0)
            ws = torch.zeros(need, dtype=torch.uint8, device=dev)
            c = sh.prepared("draft_head_lowrank", hg, Mg, g.d, GWd[i], g.r, GWu[i], g.V, sh.SH_BF16, sh.SAMPLE,
                            g.temperature, g.seeds["philox"], i, tok, lse, lp, None, ws, need,
                            torch.cuda.current_stream().cuda_stream)
            c.keep = (tok, lse, lp, ws)
            calls.append(c)
        o = run_leg("gptoss192", calls, Mg, (g.r * g.d + g.V * g.r + Mg * g.d) * 2 + Mg * 12)
        o["config"] = {"workload": g.name, "d": g.d, "V": g.V, "r": g.r, "rows": Mg, "temperature": g.temperature}
        del GWd, GWu

    # static trimmed vocabulary: the dense head over 32768 kept rows (a seeded id subset; the
    # kept rows are gathered once, as a trimmed head stores them)
    if "trimmed48" in legs or "trimmed6" in legs:
        n_keep = 32768
        keep = np.sort(np.random.default_rng(seeds["weights"] + 77).choice(V, n_keep, replace=False)).astype(np.int32)
        keep_t = torch.from_numpy(keep).to(dev)
        WS = [W.index_select(0, keep_t.long()).contiguous()]
        WS.append(WS[0].clone())
        for name, hh, M in (("trimmed48", h48, 48), ("trimmed6", h6, 6)):
            if name not in legs:
                continue
            calls = []
            for i in range(2):
                tok = torch.empty(M, dtype=torch.int32, device=dev)
                lse = torch.empty(M, dtype=torch.float32, device=dev)
                lp = torch.empty(M, dtype=torch.float32, device=dev)
                need = sh.load().sh_head_workspace_bytes(sh.OP_DENSE, M, d, 0, n_keep, 0)
                ws = torch.zeros(need, dtype=torch.uint8, device=dev)
                c = sh.prepared("draft_head_trimmed", hh, M, d, WS[i], n_keep, keep_t, sh.SH_BF16, sh.SAMPLE, 1.0,
                                seeds["philox"], i, tok, lse, lp, None, ws, need, torch.cuda.current_stream().cuda_stream)
                c.keep = (tok, lse, lp, ws)
                calls.append(c)
            o = run_leg(name, calls, M, (n_keep * d + M * d) * 2 + n_keep * 4 + M * 12)
            o["config"] = {"kept_rows": n_keep}
        del WS

    if "trimmedceiling" in legs:
        line_extra["trimmed_ceiling"] = trimmed_ceiling(sh, synth, W, V, d, seeds, dev, bf)

    # position-adaptive rank: 8 sequences x 6 draft positions with ranks falling by position
    # (nested prefixes of the r = 512 pair); "s" = every position at rank <= 256 (half the columns)
    for name, sched in (("adaptive48", [512, 512, 384, 384, 256, 256]), ("adaptive48s", [256, 256, 192, 192, 128, 128])):
        if name not in legs:
            continue
        ranks = np.array(sched * 8, dtype=np.int32)
        cols = min(r, (int(ranks.max()) + 127) // 128 * 128)
        calls = []
        for i in range(R):
            tok = torch.empty(48, dtype=torch.int32, device=dev)
            lse = torch.empty(48, dtype=torch.float32, device=dev)
            lp = torch.empty(48, dtype=torch.float32, device=dev)
            need = sh.load().sh_head_workspace_bytes(sh.OP_LOWRANK, 48, d, r, V, 0)
            ws = torch.zeros(need, dtype=torch.uint8, device=dev)
            c = sh.prepared("draft_head_lowrank_adaptive", h48, 48, d, Wd[i], r, Wu[i], V, ranks, sh.SH_BF16,
                            sh.SAMPLE, 1.0, seeds["philox"], i, tok, lse, lp, None, ws, need,
                            torch.cuda.current_stream().cuda_stream)
            c.keep = (tok, lse, lp, ws)
            calls.append(c)
        alg = (int(ranks.max()) * d + V * cols + 48 * d) * 2 + 48 * 12
        o = run_leg(name, calls, 48, alg)
        o["config"] = {"ranks_by_position": sched, "columns_read": cols}

    vsweep = [(sg, nm) for sg, nm in ((1.0, "verify"), (0.5, "verifys0.5"), (2.0, "verifys2")) if nm in legs]
    if "verifyg" in legs and not any(sg == 1.0 for sg, _ in vsweep):
        vsweep.insert(0, (1.0, None))
    for sigma, vname in vsweep:
        vw = configs.VERIFY
        inp = synth.verify_inputs(vw.B, vw.gamma, vw.V, sigma, "bf16", vw.seeds)
        tl = [bf(inp["target"])]
        dl = [bf(inp["draft"])]
        for _ in range(2):
            tl.append(tl[0].clone())
            dl.append(dl[0].clone())
        toks = torch.from_numpy(inp["tokens"]).to(dev)
        u = torch.from_numpy(inp["u"]).to(dev)
        del inp
        for name, mode in ((vname, sh.SAMPLE), ("verifyg" if sigma == 1.0 else None, sh.GREEDY)):
            if name is None or name not in legs:
                continue
            calls = []
            for i in range(3):
                acc = torch.empty(vw.B, dtype=torch.int32, device=dev)
                out = torch.empty(vw.B, vw.gamma + 1, dtype=torch.int32, device=dev)
                need = sh.load().sh_verify_workspace_bytes(mode, vw.B, vw.gamma, vw.V)
                ws = torch.zeros(need, dtype=torch.uint8, device=dev)
                c = sh.prepared("spec_verify", mode, vw.B, vw.gamma, vw.V, sh.SH_BF16, tl[i],
                                dl[i] if mode == sh.SAMPLE else None, toks, u if mode == sh.SAMPLE else None,
                                1.0, vw.seeds["philox"], i, acc, out, ws, need,
                                torch.cuda.current_stream().cuda_stream)
                c.keep = (acc, out, ws)
                calls.append(c)
            rows_bytes = vw.B * (vw.gamma + 1) * vw.V * 2 + (vw.B * vw.gamma * vw.V * 2 if mode == sh.SAMPLE else 0)
            alg = rows_bytes + vw.B * vw.gamma * 8 + vw.B * (vw.gamma + 2) * 4
            o = run_leg(name, calls, vw.B * vw.gamma, alg, "draft tokens")
            o["config"] = {"B": vw.B, "gamma": vw.gamma, "V": vw.V, "sigma": sigma}
            o["acceptance"] = acceptance_stats(calls[0].keep[0], vw.gamma)

    if "verifysparse" in legs:
        vw = configs.VERIFY
        ks = w.k   # the SpecVocab head's candidate count
        inp = synth.verify_sparse_inputs(vw.B, vw.gamma, vw.V, ks, 1.0, "bf16", vw.seeds)
        tl = [bf(inp["target"])]
        for _ in range(2):
            tl.append(tl[0].clone())
        idx = torch.from_numpy(inp["idx"]).to(dev)
        prob = torch.from_numpy(inp["prob"]).to(dev)
        toks = torch.from_numpy(inp["tokens"]).to(dev)
        u = torch.from_numpy(inp["u"]).to(dev)
        need = sh.load().sh_verify_sparse_workspace_bytes(vw.B, vw.gamma, vw.V, ks)
        calls = []
        for i in range(3):
            acc = torch.empty(vw.B, dtype=torch.int32, device=dev)
            out = torch.empty(vw.B, vw.gamma + 1, dtype=torch.int32, device=dev)
            ws = torch.zeros(need, dtype=torch.uint8, device=dev)
            c = sh.prepared("spec_verify_sparse", vw.B, vw.gamma, vw.V, ks, sh.SH_BF16, tl[i], idx, prob, toks, u,
                            1.0, vw.seeds["philox"], i, acc, out, ws, need, torch.cuda.current_stream().cuda_stream)
            c.keep = (acc, out, ws)
            calls.append(c)
        alg = vw.B * (vw.gamma + 1) * vw.V * 2 + vw.B * vw.gamma * ks * 8 + vw.B * vw.gamma * 8 + vw.B * (vw.gamma + 2) * 4
        o = run_leg("verifysparse", calls, vw.B * vw.gamma, alg, "draft tokens")
        o["config"] = {"B": vw.B, "gamma": vw.gamma, "V": vw.V, "k": ks, "sigma": 1.0}

    if "verifytree" in legs:
        vw = configs.VERIFY
        TB, TN = vw.B, 16   # 64 candidate trees of 16 nodes over the verification vocabulary
        inp = synth.tree_inputs(TB, TN, vw.V, 0.5, "bf16", vw.seeds)
        tl = [bf(inp["target"])]
        for _ in range(2):
            tl.append(tl[0].clone())
        ttok = torch.from_numpy(inp["tokens"]).to(dev)
        tpar = torch.from_numpy(inp["parent"]).to(dev)
        need = sh.load().sh_verify_tree_workspace_bytes(TB, TN, vw.V)
        calls = []
        for i in range(3):
            acc = torch.empty(TB, dtype=torch.int32, device=dev)
            node = torch.empty(TB, dtype=torch.int32, device=dev)
            out = torch.empty(TB, TN, dtype=torch.int32, device=dev)
            ws = torch.zeros(need, dtype=torch.uint8, device=dev)
            c = sh.prepared("spec_verify_tree", TB, TN, vw.V, sh.SH_BF16, tl[i], ttok, tpar, acc, node, out, ws,
                            need, torch.cuda.current_stream().cuda_stream)
            c.keep = (acc, node, out, ws)
            calls.append(c)
        alg = TB * TN * vw.V * 2 + TB * TN * 8 + TB * (TN + 2) * 4
        o = run_leg("verifytree", calls, TB * (TN - 1), alg, "candidate nodes")
        o["config"] = {"B": TB, "N": TN, "V": vw.V, "sigma": 0.5}

    head = results.get("lowrank48")
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"] if head else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_call"] if head else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) hidden states, N(0, 1/fan_in) weights)",
        "config": {"workload": w.name, "head": "slimspec-lowrank", "d": d, "V": V, "r": r,
                   "rows": 48, "sequences": 8, "gamma": 6, "mode": "sample", "temperature": 1.0,
                   "parallelism": "none (one GPU)"},
    }
    if head:
        line["hbm_roofline_frac_call"] = head["hbm_frac"]
    # roofline of the dominant kernel: the W_up streaming kernel of the headline leg
    rbw = read_bandwidth(sh, torch, dev)
    log(f"  read bandwidth (1 GiB flat read) {rbw['GBps']:.0f} GB/s")
    line["read_bandwidth"] = rbw
    for v in results.values():   # each leg's algorithmic bytes per second against the measured read rate
        v["frac_of_measured_read"] = v["alg_bytes"] / (v["ms_per_call"] / 1000.0) / (rbw["GBps"] * 1e9)
    if head and "kernels" in head:
        kname = next(k for k in ("head_tile", "head_kchunk", "head_wide", "stream_mfma", "stream_valu") if k in head["kernels"])
        kavg = head["kernels"][kname]["avg_us"]
        kbytes = V * r * 2 + 48 * r * 2   # the W_up pass: W_up and h_r
        achieved = kbytes / (kavg * 1e-6) / 1e9
        traffic = None
        if kname == "head_tile" and os.path.exists(TRAFFIC_JSON):
            t = json.load(open(TRAFFIC_JSON))
            if t.get("source_sha256") == sha_of(KERNEL_SOURCES):
                traffic = t.get("hbm_bytes_per_launch")
        line["roofline"] = {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                            "alg_bytes_per_launch": kbytes, "avg_launch_us": kavg,
                            "frac_of_measured_read": achieved / rbw["GBps"]}
    if "dense48" in results and head:
        line["nu_lowrank_vs_dense_M48"] = head["ms_per_call"] / results["dense48"]["ms_per_call"]
    if "dense6" in results and "lowrank6" in results:
        line["nu_lowrank_vs_dense_M6"] = results["lowrank6"]["ms_per_call"] / results["dense6"]["ms_per_call"]
    if "specvocab1" in results and "dense6" in results:
        line["nu_specvocab1_vs_dense6"] = results["specvocab1"]["ms_per_call"] / results["dense6"]["ms_per_call"]
    if "verify" in results:
        line["verify_tokens_per_s"] = results["verify"]["tokens_per_s"]
    if "verifysparse" in results:
        line["verify_sparse_tokens_per_s"] = results["verifysparse"]["tokens_per_s"]
    if "verifytree" in results:
        line["verify_tree_nodes_per_s"] = results["verifytree"]["tokens_per_s"]
    line.update(line_extra)
    if any(k.startswith("verify") and "acceptance" in v for k, v in results.items()):
        line["verify_sigma_sweep"] = {str(v["config"]["sigma"]): {"us_per_call": v["us_per_call"],
                                                                  "tokens_per_s": v["tokens_per_s"], **v["acceptance"]}
                                      for k, v in results.items() if "acceptance" in v and k != "verifyg"}
    line["legs"] = {kk: {x: v for x, v in vv.items() if x != "kernels"} for kk, vv in results.items()}
    line["kernels_us"] = {kk: {kn: round(kv["avg_us"], 3) for kn, kv in vv.items()} for kk, vv in kernel_trace.items()}

    if head and not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(h48_np, Wd_np, Wu_np, seeds["philox"])
    print(json.dumps(line), flush=True)


def acceptance_stats(acc_t, gamma):
    """Accepted-draft statistics of one sampling verification call: mean accepted length a,
    mean emitted tokens a + 1, the acceptance rate over attempted positions (a accepts out of
    min(a + 1, gamma) tries per sequence), and the explainer's closed form for E[a + 1] at that
    rate, (1 - alpha^(gamma + 1)) / (1 - alpha)."""
    a = acc_t.detach().cpu().numpy().astype(np.float64)
    tries = np.minimum(a + 1, gamma).sum()
    alpha = float(a.sum() / tries) if tries else 0.0
    closed = (1 - alpha ** (gamma + 1)) / (1 - alpha) if alpha < 1 else gamma + 1.0
    return {"mean_accept_len": float(a.mean()), "mean_emitted": float(a.mean() + 1), "alpha_hat": alpha,
            "closed_form_emitted_at_alpha_hat": closed}


def trimmed_ceiling(sh, synth, W, V, d, seeds, dev, bf):
    """The acceptance ceiling of a static trimmed vocabulary (SlimSpec write-up, section 二):
    a draft supported on the kept ids S can be accepted at most with probability p(S).  Target
    scores come from the dense head (the library's kernel, raw logits) for B sequences x
    (gamma + 1) positions; the drafter is the trimmed head over the same 32768 kept ids as the
    trimmed legs (its sampled tokens), with draft scores equal to the target's on S (the best a
    trimmed drafter can do: q = p restricted to S, renormalised) or with N(0, 1) noise added on S;
    both are verified by spec_verify.  Reports the mean p(S) over the attempted positions and
    the acceptance rates measured through verification."""
    import torch
    B, gamma, n_keep = 512, 5, 32768
    keep = np.sort(np.random.default_rng(seeds["weights"] + 77).choice(V, n_keep, replace=False)).astype(np.int32)
    keep_t = torch.from_numpy(keep).to(dev)
    rows = B * (gamma + 1)
    h = bf(synth.hidden(rows, d, "bf16", seeds["hidden"] + 500))
    z = torch.empty(rows, V, dtype=torch.float32, device=dev)
    for r0 in range(0, rows, 192):
        out = sh.draft_head_dense(h[r0:r0 + 192], W, want_logits=True, want_lse=False)
        z[r0:r0 + 192] = out["logits"]
    target = z.to(torch.bfloat16).view(B, gamma + 1, V).contiguous()
    del z
    lp = torch.log_softmax(target.float(), dim=-1)
    pS = torch.logsumexp(lp[:, :, keep_t.long()], dim=-1).exp()          # [B, gamma + 1]
    W_S = W.index_select(0, keep_t.long()).contiguous()
    hd = h.view(B, gamma + 1, d)[:, :gamma].reshape(B * gamma, d).contiguous()
    res = {"B": B, "gamma": gamma, "kept": n_keep, "V": V}
    gnoise = torch.Generator(device="cpu").manual_seed(seeds["weights"] + 91)
    for kind, noise in (("exact_on_S", 0.0), ("noisy_on_S", 1.0)):
        draft = torch.full((B, gamma, V), float("-inf"), dtype=torch.bfloat16, device=dev)
        ds = target[:, :gamma][:, :, keep_t.long()].float()
        if noise:
            ds = ds + noise * torch.randn(ds.shape, generator=gnoise).to(dev)
        draft[:, :, keep_t.long()] = ds.to(torch.bfloat16)
        # the drafter's tokens: sampled by the trimmed head (ids in S)
        if noise:
            # a noisy drafter samples from its own (noisy) scores: Gumbel-max over S
            g = -torch.log(-torch.log(torch.rand(ds.shape, generator=gnoise).to(dev).clamp_min(1e-12)))
            toks = keep_t[(ds + g).argmax(dim=-1)].to(torch.int32)
        else:
            toks = sh.draft_head_trimmed(hd, W_S, keep_t, mode="sample", seed=seeds["philox"], offset=7)["token"]
            toks = toks.view(B, gamma).contiguous()
        u = torch.from_numpy(synth.uniforms_open((B, gamma), seeds["philox"] + 13)).to(dev)
        acc, _ = sh.spec_verify(target, draft.contiguous(), toks.view(B, gamma).contiguous(), u, mode="sample",
                                seed=seeds["philox"], offset=3)
        a = acc.cpu().numpy().astype(np.int64)
        tried = np.minimum(a + 1, gamma)
        ps = pS[:, :gamma].cpu().numpy()
        mask = np.arange(gamma)[None, :] < tried[:, None]
        res[kind] = {"alpha_hat": float(a.sum() / tried.sum()), "p_S_mean_over_tries": float(ps[mask].mean()),
                     "tries": int(tried.sum())}
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(h, Wd, Wu, seed):
    """The oracle, as it stands, on the headline workload: full low-rank calls (48 rows, all V,
    sampling), repeated until about 12 s of host time has been spent (at most 100 calls)."""
    from oracle import heads
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count()
    n = 0
    t0 = time.time()
    while n < 100 and (time.time() - t0) < 12.0:
        heads.head_lowrank(h, Wd, Wu, "bf16", "sample", 1.0, seed, n)
        n += 1
    dt = time.time() - t0
    return {"value": 48 * n / dt, "unit": "tokens/s", "cores": threads, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{n} full oracle calls of the headline workload (48 rows x V=128256, r=512, "
                      f"sampling), {dt:.1f} s on the host"}


if __name__ == "__main__":
    main()
