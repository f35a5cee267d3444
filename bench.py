#!/usr/bin/env python3
"""Benchmark of the FlashHead two-stage retrieval head on one MI355X.

One step = one call of the head on one batch of synthetic hidden vectors:
stage-1 centroid scores, cluster selection, stage-2 candidate logits and the
decode.  Default workload: the Llama-3.2-1B head shape (v=128256, d=2048,
c=8016 clusters of b=16, p=512 probes), bf16, batch 1, greedy.

Timing
  cold (headline): before every call a 1 GiB buffer is read through the
      GPU (untimed, read-only like the weight reads of a decode step, so no
      dirty lines are left behind) so that neither L2 nor the 256 MB
      Infinity Cache holds the head's data; the call is bracketed by HIP
      events on its stream.
  warm: K back-to-back calls between two events.
  kernels: HIP events recorded exactly around each kernel by the library
      (flashhead_profile_begin/_end) during a separate cold pass.
The dense head z = E h with the same decode runs on the same GPU with the
same protocol.  The CPU oracle is timed on a bounded sample on the host.
Inputs are resident in HBM before any timed region.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "head µs/call + achieved HBM GB/s vs dense E·h, v=128256 d=2048 p=512"
HBM_PEAK_GBS = 8000.0
PAGES_TPOT_H_US = 400.0   # the paper page's Table 3 FlashHead TPOT^H (0.40 ms)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def sources_digest() -> str:
    """Digest of the library's kernel sources: counters taken on other
    sources no longer describe the kernels that run."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "two_stage_retrieval_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "flashhead.h"))
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fp:
            h.update(fp.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, B: int):
    """HBM bytes per launch of `kernel` from the rocprofv3 FETCH_SIZE and
    WRITE_SIZE runs recorded in profiles/, or None when there is no record
    for these sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    digest = sources_digest()
    for line in open(TRAFFIC_FILE):
        if not line.startswith("traffic "):
            continue
        kv = dict(item.split("=", 1) for item in line.split()[1:])
        if (kv.get("kernel") == kernel and kv.get("workload") == workload
                and int(kv.get("batch", -1)) == B and kv.get("sources") == digest):
            return int(kv["bytes"])
    return None


def algorithmic_bytes(wl, B, U, int4):
    """Bytes the method must move per call (stage 1 + candidates + io)."""
    e = 2 if wl.dtype == "bf16" else 4
    s1 = (wl.c * wl.d // 2 + wl.c * (wl.d // 128) * 2) if int4 else wl.c * wl.d * e
    stage1 = s1 + B * wl.d * e + B * wl.c * 4
    stage2 = U * wl.b * wl.d * e + U * wl.b * 4 + B * wl.d * e + B * wl.p * 4 + B * 4
    total = s1 + U * wl.b * wl.d * e + U * wl.b * 4 + B * wl.d * e + B * 4
    return total, stage1, stage2


def stream_all_bytes(wl, B, int4, with_lse):
    """Bytes the all-cluster stream moves per launch: C (or its INT4 tiles),
    every row of E with its token id, H, the stage-1 keys it writes and one
    record per (16-row item, batch row)."""
    e = 2 if wl.dtype == "bf16" else 4
    s1 = (wl.c * wl.d // 2 + wl.c * (wl.d // 128) * 2) if int4 else wl.c * wl.d * e
    rec = (wl.v // 16) * B * (16 if with_lse else 8)
    return s1 + wl.v * wl.d * e + wl.v * 4 + B * wl.d * e + B * wl.c * 4 + rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=1)
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--tau", type=float, default=1.0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--warm", action="store_true",
                    help="also time back-to-back (cache-warm) calls")
    ap.add_argument("--c", type=int, default=None, help="cluster count variant (v = c * b)")
    ap.add_argument("--b", type=int, default=None, help="cluster size variant (v = c * b)")
    ap.add_argument("--p", type=int, default=None, help="probe count variant")
    ap.add_argument("--mc", type=int, default=0, metavar="N",
                    help="time the Monte Carlo marginal (Formula 7) with N draws "
                         "instead of the decode step; prints its own JSON line")
    ap.add_argument("--mc-tokens", type=int, default=16)
    ap.add_argument("--kmeans", type=int, default=0, metavar="N",
                    help="time N iterations of the equal-size spherical k-means "
                         "(Module 1) on the workload's E instead of the decode step; "
                         "prints its own JSON line")
    ap.add_argument("--adaptive", type=float, default=0.0, metavar="EPS",
                    help="adaptive probe count: clusters whose stage-1 softmax weight is at "
                         "least EPS times the largest, clamped to [--p-min, p]")
    ap.add_argument("--p-min", type=int, default=16)
    ap.add_argument("--bf16-stage1", action="store_true",
                    help="score the centroids in bf16 even where the workload names INT4")
    ap.add_argument("--flags", type=int, default=0,
                    help="fh_desc.flags for the head (1: cooperative single launch)")
    ap.add_argument("--timeline", type=int, default=0, metavar="N",
                    help="load the measurement build (libflashhead_trace.so) and print the "
                         "median timeline of N cold batch-1 calls instead of the bench line")
    ap.add_argument("--timeline-warm", action="store_true",
                    help="with --timeline: no cache flush before the calls")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run --steps cold calls and a 256 MiB copy-like kernel, then exit "
                         "(for rocprofv3 --pmc runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(batch rows shard across GPUs with no exchange; see the design "
              "notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.timeline:
        os.environ["FLASHHEAD_LIB_VARIANT"] = "trace"
    import torch

    from two_stage_retrieval_amd import binding as fhb
    from two_stage_retrieval_amd import synth

    wl = synth.workload(args.workload)
    if args.c or args.b or args.p:
        # c / p variants of the same head shape ([paper] Table 7's trade-off)
        import dataclasses
        c = args.c or wl.c
        b = args.b or wl.b
        p = args.p or wl.p
        wl = dataclasses.replace(wl, name=f"{wl.name}-c{c}-b{b}-p{p}", c=c, b=b, v=c * b, p=p)
    B = args.batch or wl.batches[0]
    if args.bf16_stage1 and wl.quant != "none":
        import dataclasses
        wl = dataclasses.replace(wl, name=wl.name + "-bf16-stage1", quant="none")
    int4 = wl.quant == "int4_g128"
    sample = wl.mode == "sample"
    tau = args.tau if sample else 1.0
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.kmeans:
        kmeans_bench(args, wl, dev)
        return

    t0 = time.time()
    head = synth.make_head(wl)
    nvec = max(B * 64, 1024 if B == 1 else B * 8)
    H = synth.make_hidden(head, nvec)
    log(f"[bench] generated workload {wl.name} in {time.time() - t0:.1f}s")

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    E_dev = to_dev(head.E)
    H_dev = to_dev(H)
    C_init = to_dev(head.C_given) if head.C_given is not None else None
    fh = fhb.FlashHead(E_dev, head.c2t, C_init,
                       quant=fhb.FH_QUANT_INT4_G128 if int4 else fhb.FH_QUANT_NONE,
                       max_batch=B, max_p=wl.p, flags=args.flags)
    nb = nvec // B
    batches = [H_dev[i * B:(i + 1) * B] for i in range(nb)]
    out = torch.empty(B, dtype=torch.int32, device=dev)
    seeds = [torch.from_numpy(synth.make_seeds(i, B).view(np.int64)).to(dev)
             for i in range(nb)]
    flush = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def evict():
        fhb.flashhead_stream_read(flush, flush_sink)
    torch.cuda.synchronize()
    log(f"[bench] prepared in {time.time() - t0:.1f}s")

    out_p = torch.empty(B, dtype=torch.int32, device=dev)

    def call(i):
        x = batches[i % nb]
        if args.adaptive:
            if sample:
                fh.sample_adaptive(x, args.p_min, wl.p, args.adaptive, tau, seeds[i % nb],
                                   out=out, out_p=out_p)
            else:
                fh.greedy_adaptive(x, args.p_min, wl.p, args.adaptive, out=out, out_p=out_p)
        elif sample:
            fh.sample(x, wl.p, tau, seeds[i % nb], out=out)
        else:
            fh.greedy(x, wl.p, out=out)

    if args.mc:
        mc_bench(args, wl, head, H, H_dev, fh, evict, int4)
        fh.close()
        return
    if args.timeline:
        timeline_bench(args, wl, fh, call, evict, B)
        fh.close()
        return

    dense = None if args.no_dense else fhb.DenseHead(E_dev, max_batch=B)

    def call_dense(i):
        x = batches[i % nb]
        if sample:
            dense(x, fhb.FH_MODE_SAMPLE, tau, seeds[i % nb], out=out)
        else:
            dense(x, out=out)

    def time_cold(fn, K):
        ev = [(torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        torch.cuda.synchronize()
        for i in range(K):
            evict()
            ev[i][0].record()
            fn(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in ev]

    def time_warm(fn, K):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(K):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / K

    K, W = args.steps, args.warmup
    if args.pmc_probe:
        # counters per dispatch: the head's kernels on cold calls, then a
        # copy-like kernel of known size (reads and writes 256 MiB) whose
        # FETCH_SIZE / WRITE_SIZE calibrate the counters' units
        time_cold(call, K)
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        evict()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_probe": wl.name, "batch": B, "calls": K,
                          "copy_kernel_bytes_each_way": src.numel() * 4}), flush=True)
        fh.close()
        return

    # every call below, warm-up included, follows a flush, so that each
    # dispatch of the head's kernels in this process is a cold one
    time_cold(call, W)
    if dense:
        time_cold(call_dense, W)
    torch.cuda.synchronize()
    log("[bench] warmup done")

    cold = time_cold(call, K)
    warm = time_warm(call, K) if args.warm else None
    log(f"[bench] flashhead cold p50 {statistics.median(cold):.2f} us"
        + (f", warm {warm:.2f} us" if warm else ""))

    # the flush itself is a plain streaming read of 1 GiB (the library's
    # reference kernel): the read bandwidth this GPU achieves, measured in
    # the same process
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(10)]
    for a, b in ev:
        a.record()
        evict()
        b.record()
    torch.cuda.synchronize()
    stream_us = statistics.median([a.elapsed_time(b) * 1e3 for a, b in ev])
    stream_gbs = flush.numel() * 4 / (stream_us * 1e-6) / 1e9
    log(f"[bench] streaming read of 1 GiB: {stream_us:.1f} us = {stream_gbs:.0f} GB/s")

    # per-kernel durations (events around each kernel), cold
    fhb.flashhead_profile_begin(fh.handle, K)
    time_cold(call, K)
    stage_ms, ncalls = fhb.flashhead_profile_end(fh.handle)
    kern_us = [x * 1e3 for x in stage_ms]
    path = fhb.flashhead_query(fh.handle, 10)
    if path == 1:  # the whole step is one kernel: there are no separate stages to time
        log(f"[bench] kernel us: decode_b1 {kern_us[0]:.2f} over {ncalls} calls")
    elif path == 4:  # stage 1 and every cluster's records in one launch, then select + fold
        log(f"[bench] kernels us: stream_all {kern_us[0]:.2f} select_fold {kern_us[1]:.2f} "
            f"over {ncalls} calls")
    else:
        log(f"[bench] kernels us: stage1 {kern_us[0]:.2f} select {kern_us[1]:.2f} "
            f"stage2 {kern_us[2]:.2f} over {ncalls} calls")
    # a bounded wait between workgroups that gave up, or a selection of the
    # wrong size, leaves a bit in the self-check word: the timings above are
    # then of a step that did not compute the head, and no line is printed
    check = fhb.flashhead_query(fh.handle, 9)
    if check:
        log(f"[bench] FAILED: self-check word {check:#x} after the timed calls")
        sys.exit(3)

    dense_cold = dense_warm = None
    if dense:
        dense_cold = time_cold(call_dense, K)
        dense_warm = time_warm(call_dense, K) if args.warm else None
        log(f"[bench] dense cold p50 {statistics.median(dense_cold):.2f} us"
            + (f", warm {dense_warm:.2f} us" if dense_warm else ""))

    # union of selected clusters per batch (U = p at batch 1; with the
    # adaptive count, U and the bytes follow the probes each call takes)
    U = wl.p
    p_stats = None
    if args.adaptive:
        counts = []
        for i in range(nb):
            call(i)
            counts.append(out_p.cpu().numpy().copy())
        counts = np.concatenate(counts)
        p_stats = {"eps": args.adaptive, "p_min": args.p_min, "p_max": wl.p,
                   "mean": round(float(counts.mean()), 1),
                   "p10": int(np.percentile(counts, 10)), "p50": int(np.percentile(counts, 50)),
                   "p90": int(np.percentile(counts, 90)), "rows": int(len(counts))}
        log(f"[bench] adaptive probes: {p_stats}")
        if B == 1:
            U = int(round(counts.mean()))
    if B > 1:
        us = []
        for i in range(min(nb, 8)):
            dbg = {"clusters": torch.empty(B, wl.p, dtype=torch.int32, device=dev)}
            evict()
            if args.adaptive and sample:
                fh.sample_adaptive(batches[i], args.p_min, wl.p, args.adaptive, tau, seeds[i],
                                   out=out, debug=dbg)
            elif args.adaptive:
                fh.greedy_adaptive(batches[i], args.p_min, wl.p, args.adaptive, out=out,
                                   debug=dbg)
            elif sample:
                fh.sample(batches[i], wl.p, tau, seeds[i], out=out, debug=dbg)
            else:
                fh.greedy(batches[i], wl.p, out=out, debug=dbg)
            cl = dbg["clusters"].cpu().numpy()
            us.append(len(np.unique(cl[cl != 0x7FFFFFFF])))
        U = int(round(statistics.mean(us)))
    total_b, s1_b, s2_b = algorithmic_bytes(wl, B, U, int4)
    cold_p50 = statistics.median(cold)
    cold_p90 = float(np.percentile(cold, 90))
    gbs = total_b / (cold_p50 * 1e-6) / 1e9
    # dominant kernel: at batch 1 the whole step is one launch (stage 1,
    # selection, stage 2 and the decode); otherwise the longer of the two
    # streaming stages
    if path == 1:
        dom, dom_bytes, dom_name = 0, total_b, "decode_b1"
        kern_us = [kern_us[0], 0.0, 0.0]
    elif path == 4:
        # the stream reads C and every cluster's rows (not only the union)
        # and writes one record per (16-row item, batch row)
        dom, dom_name = 0, "stream_all"
        dom_bytes = stream_all_bytes(wl, B, int4, False)  # the bench asks for no lse
    elif kern_us[2] >= kern_us[0]:
        dom, dom_bytes, dom_name = 2, s2_b, "stage2"
    else:
        dom, dom_bytes, dom_name = 0, s1_b, "stage1"
    dom_gbs = dom_bytes / (kern_us[dom] * 1e-6) / 1e9
    traffic = measured_traffic(dom_name, wl.name, B)
    roofline = {"bound": "hbm", "kernel": dom_name,
                "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": dom_bytes,
                "avg_launch_us": round(kern_us[dom], 3),
                "frac_of_streaming_read": round(dom_gbs / stream_gbs, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(head, H, wl, B, int4, sample, tau, args.cpu_seconds)

    dense_p50 = statistics.median(dense_cold) if dense_cold else None
    res = {
        "metric": METRIC,
        "value": round(cold_p50, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(cold_p50 / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": (round(cold_p50 / PAGES_TPOT_H_US, 4)
                        if args.workload == 1 and B == 1 else None),
        "vs_baseline_note": "value / the paper page's FlashHead TPOT^H of 400 us "
                            "(Table 3, other hardware): context only",
        "dtype": wl.dtype if not int4 else "int4+bf16",
        "data": "synthetic (seeded generator, pages' head shapes)",
        "config": {"workload": f"{wl.name} {'sample' if sample else 'greedy'} B={B}"
                               + (f" adaptive eps={args.adaptive}" if args.adaptive else ""),
                   "v": wl.v, "d": wl.d, "c": wl.c, "b": wl.b, "p": wl.p,
                   "batch": B, "timing": "cold (1 GiB read-only flush before each call)",
                   "flags": args.flags},
        "achieved_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": total_b,
        "union_clusters": U,
        "adaptive_probes": p_stats,
        "cold_p90_us": round(cold_p90, 3),
        "warm_us": round(warm, 3) if warm else None,
        "streaming_read_gbs": round(stream_gbs, 1),
        "kernels_us": ({"decode_b1": round(kern_us[0], 3)} if path == 1 else
                       {"stream_all": round(kern_us[0], 3),
                        "select_fold": round(kern_us[1], 3)} if path == 4 else
                       {"stage1": round(kern_us[0], 3), "select": round(kern_us[1], 3),
                        "stage2": round(kern_us[2], 3)}),
        "path": path,
        "dense_us_cold": round(dense_p50, 3) if dense_p50 else None,
        "dense_us_warm": round(dense_warm, 3) if dense_warm else None,
        "speedup_vs_dense": round(dense_p50 / cold_p50, 3) if dense_p50 else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    fh.close()
    print(json.dumps(res), flush=True)


# events of the single-launch decode's measurement build (fh_trace.h)
_TL_BLOCK = {"start": 0, "keys_seen": 1, "sel_published": 2, "s2_entries": 3,
             "partial_published": 4, "token": 5, "end": 6}
_TL_WAVE = {"s1_issued": 0, "s1_done": 1, "s2_done": 2}
_TL_SEL_POINTS = (0, 2, 3, 4, 5, 6, 7)


def parse_timeline(words, khz):
    """µs from the first workgroup's start for each event of one launch."""
    nb, nw = 512, 8192
    blk = words[:8 * nb].reshape(8, nb).astype(np.int64)
    wav = words[8 * nb:8 * nb + 4 * nw].reshape(4, nw).astype(np.int64)
    sel = words[8 * nb + 4 * nw:8 * nb + 4 * nw + 32].reshape(16, 2).astype(np.int64)
    cnt = words[8 * nb + 4 * nw + 32:8 * nb + 4 * nw + 48].astype(np.int64)
    grid = int(np.count_nonzero(blk[0]))
    t0 = blk[0][:grid].min()
    us = lambda t: (t - t0) * 1e3 / khz  # noqa: E731
    waves = wav[:, :grid * 8]
    out = {"grid": grid,
           "last_workgroup_start": us(blk[0][:grid].max()),
           "stage1_requests_issued_all": us(waves[0][waves[0] > 0].max()),
           "stage1_done_median_wave": us(np.median(waves[1][waves[1] > 0])),
           "stage1_done_all": us(waves[1][waves[1] > 0].max()),
           "keys_seen_by_wg0": us(blk[1][0]),
           "selection_published": us(blk[2][0]),
           "stage2_entries_all": us(blk[3][1:grid].max()) if grid > 1 else None,
           "stage2_done_median_wave": us(np.median(waves[2][waves[2] > 0])),
           "stage2_done_all": us(waves[2][waves[2] > 0].max()),
           "partials_published_all": us(blk[4][1:grid].max()) if grid > 1 else None,
           "token_written": us(blk[5][0]),
           "last_workgroup_end": us(blk[6][:grid].max())}
    pts = [sel[i] for i in _TL_SEL_POINTS]
    out["selection_phase_cycles"] = [int(pts[i + 1][0] - pts[i][0]) for i in range(len(pts) - 1)]
    out["selection_cycles"] = int(pts[-1][0] - pts[0][0])
    sel_rt = lambda i: us(sel[i][1]) if sel[i][1] else None  # noqa: E731
    out["wg0_stage1_done"] = us(wav[1][:8][wav[1][:8] > 0].max())
    out["wg0_keys_in_registers"] = us(blk[7][0])
    out["wg0_last_reload_issued"] = sel_rt(11)
    out["early_part_published"] = sel_rt(12)
    out["boundary_gather_cycles"] = (int(sel[8][0] - sel[4][0]) if sel[8][0] else None)
    out["boundary_gathered_cycles"] = (int(sel[9][0] - sel[8][0]) if sel[9][0] else None)
    out["boundary_ranked_cycles"] = (int(sel[10][0] - sel[9][0]) if sel[10][0] else None)
    lags = []
    for b in range(1, grid):
        w2 = wav[2][b * 8:(b + 1) * 8]
        w2 = w2[w2 > 0]
        if blk[4][b] and len(w2):
            lags.append((blk[4][b] - w2.max()) * 1e3 / khz)
    out["publish_lag_median"] = float(np.median(lags)) if lags else None
    out["publish_lag_max"] = float(np.max(lags)) if lags else None
    last = int(np.argmax(blk[4][:grid]))
    w2l = wav[2][last * 8:(last + 1) * 8]
    out["last_publisher_stage2_done"] = us(w2l[w2l > 0].max()) if (w2l > 0).any() else None
    # the workgroup whose stage 2 ends last: its index, when its entries
    # arrived, and how many workgroups got their entries after the first
    # selection publication
    done_wg = np.array([wav[2][b * 8:(b + 1) * 8].max() for b in range(grid)])
    lw = int(np.argmax(done_wg))
    out["last_stage2_workgroup"] = lw
    out["last_stage2_workgroup_entries"] = us(blk[3][lw]) if lw > 0 and blk[3][lw] else None
    out["last_stage2_workgroup_share_us"] = (us(done_wg[lw]) - us(blk[3][lw])
                                             if lw > 0 and blk[3][lw] else None)
    ent = blk[3][1:grid]
    out["entries_after_full_selection"] = int(np.count_nonzero(ent > blk[2][0])) if blk[2][0] else None
    out["key_poll_rounds"] = int(cnt[0])
    out["merge_poll_rounds"] = int(cnt[1])
    out["boundary_bin_keys"] = int(cnt[2])
    return out


def timeline_bench(args, wl, fh, call, evict, B):
    """The median over N cold calls of each event of the single-launch decode
    (the measurement build's timestamps), as one JSON line."""
    import torch

    from two_stage_retrieval_amd import binding as fhb
    if B != 1:
        raise SystemExit("--timeline times the single-launch batch-1 decode (--batch 1)")
    fhb.flashhead_trace_read()  # clear
    runs = []
    for i in range(args.timeline + 5):
        if not args.timeline_warm:
            evict()
        call(i)
        torch.cuda.synchronize()
        words, khz = fhb.flashhead_trace_read()
        if i >= 5:
            runs.append(parse_timeline(words, khz))
    if fhb.flashhead_query(fh.handle, 10) != 1:
        raise SystemExit("the step did not take the single launch")
    check = fhb.flashhead_query(fh.handle, 9)
    if check:
        raise SystemExit(f"self-check word {check:#x}")
    med = {}
    for k, v in runs[0].items():
        if isinstance(v, list):
            med[k] = [int(statistics.median(r[k][j] for r in runs)) for j in range(len(v))]
            continue
        vals = [r[k] for r in runs if r[k] is not None]  # an event a launch did not reach
        med[k] = round(float(statistics.median(vals)), 3) if vals else None
    log("[bench] timeline (us from the first workgroup's start, median of "
        f"{len(runs)} cold calls):")
    for k, v in med.items():
        log(f"    {k:32s} {v}")
    import collections
    lastw = collections.Counter(r["last_stage2_workgroup"] for r in runs).most_common(4)
    log(f"    {'last_stage2_workgroup (count)':32s} {lastw}")
    print(json.dumps({"timeline": wl.name, "calls": len(runs), "median": med,
                      "last_stage2_workgroups": lastw,
                      "cache": "warm" if args.timeline_warm else "cold (1 GiB flush)",
                      "build": "libflashhead_trace.so"}), flush=True)


def mc_bench(args, wl, head, H, H_dev, fh, evict, int4):
    """Formula 7: one estimate = N draws of the probed clusters for one
    hidden vector and the mean conditional probability of Q query tokens.
    Cold timing as for the decode step; the oracle is timed on a bounded
    number of draws and scaled to N."""
    import torch
    N, Q = args.mc, args.mc_tokens
    dev = H_dev.device
    tau = args.tau
    rng = np.random.default_rng(5)
    nvec = min(len(H), 64)
    toks = [torch.from_numpy(rng.integers(0, wl.v, size=Q).astype(np.int32)).to(dev)
            for _ in range(nvec)]
    seeds = torch.from_numpy((np.arange(N, dtype=np.uint64) + (np.uint64(21) << np.uint64(32)))
                             .view(np.int64)).to(dev)
    out = torch.empty(Q, dtype=torch.float32, device=dev)
    from two_stage_retrieval_amd import binding as fhb
    nbytes = fhb.flashhead_mc_workspace_bytes(fh.handle, N, wl.p, Q)
    raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
    ws = raw[(-raw.data_ptr()) % 256:][:nbytes]

    def call(i):
        fh.mc_marginal(H_dev[i % nvec:i % nvec + 1], wl.p, tau, seeds, toks[i % nvec],
                       out=out, workspace=ws)
    times = []
    for i in range(args.warmup + args.steps):
        evict()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call(i)
        b.record()
        torch.cuda.synchronize()
        if i >= args.warmup:
            times.append(a.elapsed_time(b) * 1e3)
    us = statistics.median(times)
    log(f"[bench] mc: {N} draws, {Q} tokens: cold p50 {us:.1f} us")
    check = fhb.flashhead_query(fh.handle, 9)
    if check:
        log(f"[bench] FAILED: self-check word {check:#x} after the timed calls")
        sys.exit(3)
    if args.pmc_probe:
        # the copy-like kernel of known size that calibrates the counters
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        evict()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_probe": wl.name, "mc_draws": N, "calls": len(times),
                          "copy_kernel_bytes_each_way": src.numel() * 4}), flush=True)
        return

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import flashhead_ref as ref
        rows = ref.rows_accessor(head.E, wl.dtype)
        C64 = (ref.as_f64(head.C_given, wl.dtype) if head.C_given is not None
               else ref.centroid_means(rows, head.c2t))
        kw = {"int4": ref.int4_quantize(C64)} if int4 else {"C_f64": C64}
        h64 = ref.as_f64(H[0], wl.dtype)
        n_s = max(1, min(N, 64))
        sd = [int(x) for x in (np.arange(n_s, dtype=np.uint64) + (np.uint64(21) << np.uint64(32)))]
        t0 = time.perf_counter()
        ref.mc_marginal(rows, head.c2t, h64, wl.p, tau, sd,
                        rng.integers(0, wl.v, size=Q), **kw)
        per_draw = (time.perf_counter() - t0) * 1e6 / n_s
        cpu = {"value": round(per_draw * N, 1), "unit": "us/estimate", "cores": blas_threads(),
               "kind": "oracle",
               "sample": f"{n_s} draws timed ({per_draw:.0f} us/draw, float64 numpy oracle), "
                         f"scaled to {N} draws"}
        log(f"[bench] oracle: {per_draw:.0f} us per draw")
    res = {"metric": f"Monte Carlo marginal (Formula 7) us/estimate, {N} draws, {Q} tokens",
           "value": round(us, 3), "unit": "us/estimate", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": False,
           "dtype": wl.dtype if not int4 else "int4+bf16",
           "data": "synthetic (seeded generator, pages' head shapes)",
           "config": {"workload": f"{wl.name} mc N={N} Q={Q}", "p": wl.p, "tau": tau,
                      "timing": "cold (1 GiB read-only flush before each call)"},
           "us_per_draw": round(us / N, 4), "cpu_baseline": cpu}
    print(json.dumps(res), flush=True)


def kmeans_bench(args, wl, dev):
    """Module 1: equal-size spherical k-means of the workload's E into its c
    clusters, N assignment + update iterations from c drawn token ids.  The
    call is blocking (its rounds synchronise with the host), so it is timed
    with the host clock.  The oracle is timed for one iteration on a smaller
    head of the same generator and scaled by the (token, cluster) pairs,
    which its cosine product and pair ordering grow with."""
    import torch

    from two_stage_retrieval_amd import binding as fhb
    from two_stage_retrieval_amd import synth
    N = args.kmeans
    t0 = time.time()
    head = synth.make_head(wl)
    E = head.E
    if E.dtype == np.uint16:
        E_dev = torch.from_numpy(E.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        E_dev = torch.from_numpy(E).to(dev)
    init = np.random.default_rng(41).choice(wl.v, size=wl.c, replace=False).astype(np.int32)
    c2t = torch.empty((wl.c, wl.b), dtype=torch.int32, device=dev)
    log(f"[bench] kmeans input {wl.name} in {time.time() - t0:.1f}s")
    fhb.flashhead_kmeans(E_dev, wl.c, init, 1, c2t)  # warm-up (code, allocator)
    torch.cuda.synchronize()
    t = time.perf_counter()
    iters = fhb.flashhead_kmeans(E_dev, wl.c, init, N, c2t)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t) * 1e3
    log(f"[bench] kmeans: {iters} iterations in {ms:.1f} ms")
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import flashhead_ref as ref
        cs, bs = 512, wl.b
        small = synth.make_head(wl, c=cs, b=bs)
        rows = ref.as_f64(small.E, wl.dtype)
        init_s = np.random.default_rng(41).choice(cs * bs, size=cs, replace=False)
        t = time.perf_counter()
        ref.kmeans_equal_size(rows, cs, init_s, 1)
        sec = time.perf_counter() - t
        scale = (wl.v * wl.c) / (cs * bs * cs)
        cpu = {"value": round(sec * 1e3 * scale, 1), "unit": "ms/iteration", "cores": blas_threads(),
               "kind": "oracle",
               "sample": f"one iteration at v={cs * bs}, c={cs}, d={wl.d} ({sec:.2f} s, "
                         f"float64 numpy oracle) scaled by the pair count v*c ({scale:.0f}x)"}
        log(f"[bench] oracle: {sec:.2f} s for one iteration at v={cs * bs}, c={cs}")
    res = {"metric": "equal-size spherical k-means ms/iteration (cosines, assignment, update)",
           "value": round(ms / iters, 3), "unit": "ms/iteration", "n_gpus": 1,
           "steps": iters, "warmup": 1, "higher_is_better": False, "dtype": "f64",
           "data": "synthetic (seeded generator, pages' head shapes)",
           "config": {"workload": f"{wl.name} kmeans v={wl.v} d={wl.d} c={wl.c} b={wl.b}",
                      "iterations": iters, "timing": "host clock around the blocking call"},
           "cpu_baseline": cpu}
    print(json.dumps(res), flush=True)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads() -> int:
    """Threads of the host BLAS pool the oracle's NumPy calls use."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except ImportError:
        return int(os.environ.get("OMP_NUM_THREADS", "1"))


def cpu_baseline(head, H, wl, B, int4, sample, tau, seconds):
    """The oracle as it stands, on the host cores, over a bounded sample:
    median time of one head call (B rows), with the BLAS thread pool at its
    default size and again limited to one thread."""
    from oracle import flashhead_ref as ref
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:
        threadpool_info = threadpool_limits = None
    cores = (max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
             if threadpool_info else int(os.environ.get("OMP_NUM_THREADS", "1")))
    t0 = time.time()
    rows = ref.rows_accessor(head.E, wl.dtype)
    if head.C_given is not None:
        C64 = ref.as_f64(head.C_given, wl.dtype)
    else:
        C64 = ref.centroid_means(rows, head.c2t)
    q4 = ref.int4_quantize(C64) if int4 else None
    log(f"[bench] oracle prepare {time.time() - t0:.1f}s")
    H64 = ref.as_f64(H, wl.dtype)

    def run(budget):
        times = []
        start = time.time()
        n = 0
        while time.time() - start < budget and n < len(H64):
            t = time.perf_counter()
            for r in range(B):
                ref.flashhead_step(rows, head.c2t, H64[(n * B + r) % len(H64)], wl.p,
                                   C_f64=C64, int4=q4, mode="sample" if sample else "greedy",
                                   tau=tau, seed=r)
            times.append((time.perf_counter() - t) * 1e6)
            n += 1
        return statistics.median(times), n

    med, n = run(seconds)
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            one, n1 = run(seconds / 3)
    log(f"[bench] oracle {med:.0f} us/call on {cores} threads ({n} calls)"
        + (f", {one:.0f} us/call on 1 thread ({n1} calls)" if one else ""))
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": round(med, 1), "unit": "us/call", "cores": cores, "kind": "oracle",
            "sample": f"{n} calls of batch {B} on the same workload (float64 numpy oracle, "
                      f"{seconds:.0f} s budget), median per call",
            "value_1_thread": round(one, 1) if one else None,
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
            "affinity_cpus": affinity}


if __name__ == "__main__":
    main()
