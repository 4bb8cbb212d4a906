#!/usr/bin/env python3
"""TBE forward + backward (row-wise Adagrad) throughput on one MI355X.

One step = tbe_forward + tbe_backward_rowwise_adagrad (which runs the whole
preprocessing: transposition, radix sort, run-length encoding, classification)
over one batch of the workload; inputs are resident in HBM before timing.
Prints one JSON line with lookups/s, the roofline of the dominant kernel and
the single-threaded CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--steps K] [--warmup W] [--config C2] [--fused] [--bwd-hist]
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

METRIC = "TBE fwd+bwd lookups/sec and achieved HBM GB/s (% of MI355X peak)"
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = {
    "fwd_pool": "fwd_pool.hip", "fwd_hist": "fwd_hist.hip", "bwd_single": "bwd.hip",
    "bwd_tiny": "bwd.hip", "bwd_medium": "bwd.hip", "bwd_chunk": "bwd.hip",
    "bwd_long_update": "bwd.hip", "bwd_chunk_fused": "bwd.hip", "chunk_order": "bwd.hip",
    "bwd_hist_partial": "bwd_hist.hip", "bwd_hist_update": "bwd_hist.hip",
    "validate_check": "validate.hip",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="C2", choices=["C1", "C2", "C3", "C4", "C5"])
    ap.add_argument("--fused", action="store_true", help="fused long-run countdown path")
    ap.add_argument("--validate", action="store_true",
                    help="run tbe_validate (check only) at the start of every step")
    ap.add_argument("--bwd-hist", action="store_true",
                    help="histogram-reuse backward (one small table: C4), no preprocessing")
    ap.add_argument("--schedule", default="serial", choices=["overlap", "fork", "auto", "serial"],
                    help="overlap: tbe_preprocess on a side stream during tbe_forward, then "
                         "tbe_backward_rowwise_adagrad on preprocessed data with its run "
                         "classes on three streams; fork: tbe_forward, then "
                         "tbe_backward_rowwise_adagrad (which preprocesses) with its run classes "
                         "on three streams; auto: fork below 64 Mi lookups, else serial; "
                         "serial: all on one stream")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-lookups", type=int, default=3_000_000,
                    help="cap on lookups in the CPU oracle sample (whole tables)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


# ------------------------------------------------------------------ inputs

def device_inputs(spec, torch):
    """Index structure from the seeded numpy generators; weights, grads and
    per-sample weights drawn on the device with seeded torch generators."""
    dev = "cuda"
    off = spec.offsets()
    idx = spec.indices()
    d_off = torch.from_numpy(off).to(dev)
    d_idx = torch.from_numpy(idx).to(dev)
    wd = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[spec.wdtype]
    W, M = [], []
    for t in range(spec.T):
        g = torch.Generator(device=dev).manual_seed(spec.seed * 1000 + 500 + t)
        w = torch.rand((spec.rows[t], spec.dims[t]), generator=g, device=dev) * 0.2 - 0.1
        W.append(w.to(wd).contiguous())
        M.append(torch.zeros(spec.rows[t], dtype=torch.float32, device=dev))
    g = torch.Generator(device=dev).manual_seed(spec.seed * 1000 + 400)
    G = torch.randn((spec.B, spec.dtot), generator=g, device=dev)
    psw = None
    if spec.weighted:
        g = torch.Generator(device=dev).manual_seed(spec.seed * 1000 + 300)
        psw = torch.rand(int(off[-1]), generator=g, device=dev)
    return off, idx, d_off, d_idx, W, M, G, psw


# --------------------------------------------------------------- byte model

SL_CLASSES = (("single", 1, 2), ("tiny", 2, 32), ("medium", 32, 256), ("long", 256, None))


def workload_stats(spec, off, idx):
    """Per-table lookups, unique rows and the run-length classes the backward
    splits runs into (host, from the inputs)."""
    B = spec.B
    st = []
    for t in range(spec.T):
        lo, hi = int(off[t * B]), int(off[(t + 1) * B])
        _, cnt = np.unique(idx[lo:hi], return_counts=True)
        s = dict(n=hi - lo, U=int(cnt.size), D=spec.dims[t], mean=spec.pooling[t] == 1)
        for name, a, b in SL_CLASSES:
            m = (cnt >= a) if b is None else ((cnt >= a) & (cnt < b))
            s["n_" + name] = int(m.sum())
            s["N_" + name] = int(cnt[m].sum())
        s["chunks"] = int(((cnt[cnt >= 256] + 255) // 256).sum())
        st.append(s)
    return st


def byte_model(spec, st, hist_path):
    """Compulsory bytes per kernel family per step: each stream read or written
    once and each unique weight row once (a lower bound on HBM traffic), and the
    logical bytes of every access the method makes."""
    si = 4 if spec.itype == "i32" else 8
    sw = 4 if spec.wdtype == "f32" else 2
    psi = 1 if spec.weighted else 0
    sc = 1 if (spec.weighted or any(p == 1 for p in spec.pooling)) else 0
    T, B = spec.T, spec.B
    N = sum(s["n"] for s in st)
    U = sum(s["U"] for s in st)
    ntiles = -(-N // 4096)
    # radix passes sort the rows of each table's segment: bits of the largest table
    row_bits = max(int(np.ceil(np.log2(r))) if r > 1 else 0 for r in spec.rows)
    # the fewest passes of at most 10-bit digits, then the narrower digit of
    # 8 or 10 bits covering the rows in that many passes (as the library)
    bits = max(1, row_bits)
    w = -(-bits // -(-bits // 10))
    digit_bits = 8 if w <= 8 else 10
    npass = -(-bits // digit_bits)
    R = 1 << digit_bits
    stiles = sum(-(-s["n"] // 4096) for s in st)  # sort tiles: one table per tile
    out_bytes = B * spec.dtot * 4
    G_bytes = B * spec.dtot * 4
    comp, logi = {}, {}
    if hist_path:
        E, D = spec.rows[0], spec.dims[0]
        comp["fwd_hist"] = N * si + (B + 1) * si + E * D * sw + out_bytes
        logi["fwd_hist"] = N * si + (B + 1) * si + N * D * sw + out_bytes
    else:
        comp["fwd_pool"] = (N * (si + 4 * psi) + (T * B + 1) * si + out_bytes
                            + sum(s["U"] * s["D"] * sw for s in st))
        logi["fwd_pool"] = (N * (si + 4 * psi) + (T * B + 1) * si + out_bytes
                            + sum(s["n"] * s["D"] * sw for s in st))
    rec = 8 + 4 * sc  # sorted key + bag id (+ contribution scale)
    n = {c: sum(s["n_" + c] for s in st) for c, _, _ in SL_CLASSES}
    n_chunks = sum(s["chunks"] for s in st)
    ncls = -(-N // 2048)
    nrle = -(-N // (16384 if N >= (64 << 20) else 4096))  # run-length tiles
    st_words = nrle + ncls * 8  # look-back status words of rle and classify
    # the transposition's workgroup 0 also writes the segment table and tile map
    comp["transpose"] = (N * (si + 4 * psi) + (T * B + 1) * si + N * rec
                         + 2 * T * si + 16 * T + 4 * stiles)
    # per pass: the keys read once for the digit counts (the first pass also
    # clears the status words); the counts scanned in place; the records read
    # and written once by the scatter, plus each tile's 2^b prefixes
    comp["radix_upsweep"] = npass * (4 * N + R * 4 * stiles) + 8 * st_words
    comp["radix_scan"] = npass * 2 * R * 4 * stiles
    comp["radix_downsweep"] = npass * (2 * rec * N + R * 4 * stiles)
    comp["rle"] = 4 * N + 8 * U + 4 + 16 * nrle
    comp["classify"] = (8 * U + 4 + 4 * n["single"] + 16 * (U + n_chunks) + 8 * n["long"]
                        + 16 * 8 * ncls)
    for k in list(comp):
        logi.setdefault(k, comp[k])
    per_lookup = 4 + 4 * sc  # sorted bag id (+ scale)
    c = {k: 0.0 for k in ("bwd_single", "bwd_tiny", "bwd_medium", "bwd_chunk",
                          "bwd_long_update")}
    lg = dict(c)
    for s in st:
        D = s["D"]
        rmw = 2 * D * sw + 8  # weight row and momentum, read and written once
        for cls, kern in (("single", "bwd_single"), ("tiny", "bwd_tiny"),
                          ("medium", "bwd_medium")):
            runs, lk = s["n_" + cls], s["N_" + cls]
            g_share = G_bytes * lk / max(N, 1)
            meta = 16 * runs + (4 * sc * lk if cls == "single" else per_lookup * lk)
            c[kern] += meta + g_share + runs * rmw
            lg[kern] += meta + lk * 4 * D + runs * rmw
        lk, ch = s["N_long"], s["chunks"]
        c["bwd_chunk"] += 16 * ch + per_lookup * lk + G_bytes * lk / max(N, 1) + 4 * ch * D
        lg["bwd_chunk"] += 16 * ch + per_lookup * lk + 4 * D * lk + 4 * ch * D
        upd = 20 * s["n_long"] + 4 * ch * D + s["n_long"] * rmw
        c["bwd_long_update"] += upd
        lg["bwd_long_update"] += upd
    comp.update(c)
    logi.update(lg)
    # histogram-reuse backward (one table): indices, offsets, (per-sample weights),
    # grad_out once, the partials written and read once, each touched row updated
    if T == 1:
        D, E = spec.dims[0], spec.rows[0]
        nwg = min(1024, -(-B // 128))
        comp["bwd_hist_partial"] = (N * (si + 4 * psi) + (B + 1) * si + B * D * 4
                                    + nwg * E * (D + 1) * 4)
        comp["bwd_hist_update"] = nwg * E * (D + 1) * 4 + U * (2 * D * sw + 8)
        logi["bwd_hist_partial"] = comp["bwd_hist_partial"]
        logi["bwd_hist_update"] = comp["bwd_hist_update"]
    comp["validate_clear"] = 16
    comp["validate_check"] = N * si + (T * B + 1) * si + 16
    comp["bwd_chunk_fused"] = c["bwd_chunk"] + c["bwd_long_update"]
    logi["bwd_chunk_fused"] = lg["bwd_chunk"] + lg["bwd_long_update"]
    return comp, logi


def source_hash(kernel):
    f = KERNEL_SOURCES.get(kernel)
    if f is None:
        f = "prep.hip"
    d = os.path.join(ROOT, "table_embedding_amd", "csrc")
    h = hashlib.sha256()
    for name in (f, "tbe_common.h"):  # the kernel's file and the shared device helpers
        h.update(open(os.path.join(d, name), "rb").read())
    return h.hexdigest()[:16]


def counter_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        e = d[workload][kernel]
    except (KeyError, ValueError):
        return None
    if e.get("source_sha256_16") != source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


# ---------------------------------------------------------------- CPU leg

def cpu_baseline(spec, off, idx, W_dev, G_dev, psw_dev, cap, torch):
    """The oracle (single-threaded C) on whole tables of the same workload."""
    import oracle
    B = spec.B
    tables, n = [], 0
    for t in range(spec.T):
        nt = int(off[(t + 1) * B] - off[t * B])
        if tables and n + nt > cap:
            break
        tables.append(t)
        n += nt
    sub = [t for t in tables]
    rows = [spec.rows[t] for t in sub]
    dims = [spec.dims[t] for t in sub]
    pooling = [spec.pooling[t] for t in sub]
    lo, hi = int(off[sub[0] * B]), int(off[(sub[-1] + 1) * B])
    o = (off[sub[0] * B:(sub[-1] + 1) * B + 1].astype(np.int64) - lo).astype(off.dtype)
    ix = idx[lo:hi]
    col = spec.col_offsets()
    c0, c1 = int(col[sub[0]]), int(col[sub[-1]]) + spec.dims[sub[-1]]
    G = np.ascontiguousarray(G_dev[:, c0:c1].cpu().numpy())
    psw = None if psw_dev is None else psw_dev[lo:hi].cpu().numpy()

    def host(w):
        w = w.detach().cpu()
        return w.numpy().copy() if spec.wdtype == "f32" else w.view(torch.int16).numpy().view(np.uint16).copy()

    W = [host(W_dev[t]) for t in sub]
    M = [np.zeros(spec.rows[t], np.float32) for t in sub]
    oracle.build(force=False)
    t0 = time.perf_counter()
    oracle.forward(rows, dims, pooling, spec.wdtype, W, B, spec.itype, ix, o, psw)
    oracle.backward_rowwise_adagrad(rows, dims, pooling, spec.wdtype, W, M, B, spec.itype, ix, o,
                                    psw, G, spec.lr, spec.eps)
    dt = time.perf_counter() - t0
    return {"value": (hi - lo) / dt, "unit": "lookups/s", "cores": 1, "kind": "oracle",
            "sample": f"tables {sub[0]}..{sub[-1]} of {spec.T} ({hi - lo} lookups, all {B} bags), "
                      f"one forward + backward pass, {dt:.2f} s on 1 of {os.cpu_count()} host "
                      f"threads"}


# -------------------------------------------------------------------- main

def calibrate_copy(torch):
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n, "launches": 3}))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only (no multi-GPU path); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import table_embedding_amd as te
    import tbe_workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    te.lib()  # fail loudly if the HIP library is missing
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    spec = wl.config(args.config)
    print(f"[bench] generating {args.config}: {wl.DESCRIPTIONS[args.config]}", file=sys.stderr,
          flush=True)
    off, idx, d_off, d_idx, W, M, G, psw = device_inputs(spec, torch)
    N = int(off[-1])
    tb = te.TBE(spec.rows, spec.dims, spec.pooling, W, M)
    ws = tb.workspace(spec.B, N)
    out = torch.empty((spec.B, spec.dtot), dtype=torch.float32, device="cuda")
    flags = (te.TBE_BWD_FUSED_LONG if args.fused else 0) | (te.TBE_BWD_HIST if args.bwd_hist else 0)
    overlap = args.schedule == "overlap"
    conc = {"serial": 0, "auto": te.TBE_BWD_CONCURRENT_AUTO}.get(args.schedule,
                                                                te.TBE_BWD_CONCURRENT)
    hist = (spec.T == 1 and spec.rows[0] <= 64 and 64 <= spec.dims[0] <= 128
            and spec.wdtype == "f16" and not spec.weighted and N >= 64 * spec.B)

    err = torch.zeros(te.TBE_VALIDATE_WORDS, dtype=torch.int32, device="cuda")

    def step():
        if args.validate:
            te.tbe_validate(tb.plan, spec.B, d_idx, d_off, N, err)
        if overlap:
            tb.forward_and_preprocess(spec.B, d_idx, d_off, psw, out)
            te.tbe_backward_rowwise_adagrad(tb.plan, spec.B, d_idx, d_off, N, psw, G, spec.lr,
                                            spec.eps, ws, flags | conc | te.TBE_BWD_PREPROCESSED)
        else:
            te.tbe_forward(tb.plan, spec.B, d_idx, d_off, N, psw, out)
            te.tbe_backward_rowwise_adagrad(tb.plan, spec.B, d_idx, d_off, N, psw, G, spec.lr,
                                            spec.eps, ws, flags | conc)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps), timing {args.steps}", file=sys.stderr,
          flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # per-kernel durations: start/stop events bound to each dispatch
    te.tbe_prof_enable(True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_prof = e0.elapsed_time(e1) / args.steps
    prof = te.tbe_prof_read()
    # the per-launch floor: empty kernels timed the same way (reported only)
    te.tbe_prof_calibrate(200)
    torch.cuda.synchronize()
    n_e, t_e = te.tbe_prof_read()["empty"]
    empty_us = 1000 * t_e / n_e
    te.tbe_prof_enable(False)

    st = workload_stats(spec, off, idx)
    comp, logi = byte_model(spec, st, hist)
    kernels = {}
    for k, (n, tot) in prof.items():
        # kernel time = the dispatch's end minus its begin timestamp
        kern_us = max(1000 * tot / n, 1e-3)
        per_step_ms = kern_us * n / args.steps / 1000
        kernels[k] = {"launches_per_step": n / args.steps, "ms_per_step": round(per_step_ms, 5),
                      "avg_launch_us": round(kern_us, 3),
                      "compulsory_bytes_per_step": int(comp.get(k, 0)),
                      "gbs_compulsory": round(comp.get(k, 0) / (per_step_ms * 1e6), 1)}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom]
    launches = dk["launches_per_step"]
    bytes_per_launch = comp.get(dom, 0) / launches
    achieved = bytes_per_launch / (dk["avg_launch_us"] * 1e3)  # GB/s
    pmc_key = args.config + ("_hist" if args.bwd_hist else "")
    traffic = counter_traffic(dom, pmc_key)
    step_comp = sum(comp[k] for k in kernels if k in comp)
    # counter-measured HBM bytes of the whole step: every kernel's committed
    # FETCH_SIZE + WRITE_SIZE per launch (calibrated) times its launches per
    # step; null unless every kernel's counters were taken on its current source
    per_kernel = {k: counter_traffic(k, pmc_key) for k in kernels}
    step_counter = (sum(per_kernel[k] * kernels[k]["launches_per_step"] for k in kernels)
                    if kernels and all(v is not None for v in per_kernel.values()) else None)
    step_logi = sum(logi[k] for k in kernels if k in logi)
    lookups_s = N / (ms / 1e3)
    res = {
        "metric": METRIC,
        "value": round(lookups_s, 1),
        "unit": "lookups/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.wdtype,
        "data": "synthetic (seeded Zipf / uniform indices, device-drawn weights and grads)",
        "config": {"workload": args.config, "description": wl.DESCRIPTIONS[args.config],
                   "lookups": N, "tables": spec.T, "bags_per_table": spec.B,
                   "index_type": spec.itype, "long_run_path": "fused" if args.fused else
                   "two-launch", "schedule": args.schedule,
                   "backward": "histogram-reuse contraction" if args.bwd_hist else "run pipeline",
                   "input_validation": bool(args.validate),
                   "step": {"overlap": "tbe_forward || tbe_preprocess (side stream), then "
                                       "tbe_backward_rowwise_adagrad(PREPROCESSED) with medium "
                                       "runs and long runs on two side streams",
                            "fork": "tbe_forward, then tbe_backward_rowwise_adagrad "
                                    "(preprocessing inside) with medium runs and long runs on "
                                    "two side streams",
                            "auto": "as fork below 64 Mi lookups, else as serial "
                                    "(TBE_BWD_CONCURRENT_AUTO)",
                            "serial": "tbe_forward, then tbe_backward_rowwise_adagrad "
                                      "(preprocessing inside), one stream"}[args.schedule]},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "hbm": {"compulsory_bytes_per_step": int(step_comp),
                "achieved_gbs_compulsory": round(step_comp / (ms * 1e6), 1),
                "frac_of_peak_compulsory": round(step_comp / (ms * 1e6) / HBM_PEAK_GBS, 4),
                "logical_bytes_per_step": int(step_logi),
                "effective_gbs_logical": round(step_logi / (ms * 1e6), 1),
                "counter_bytes_per_step": None if step_counter is None else int(step_counter),
                "counter_gbs": None if step_counter is None else
                round(step_counter / (ms * 1e6), 1),
                "counter_frac_of_peak": None if step_counter is None else
                round(step_counter / (ms * 1e6) / HBM_PEAK_GBS, 4),
                "traffic_ratio": None if step_counter is None or not step_comp else
                round(step_counter / step_comp, 3),
                "counter_source": "profiles/pmc_traffic.json (rocprofv3 FETCH_SIZE x2.000 + "
                                  "WRITE_SIZE x1.000 per launch, serial schedule)"},
        "kernel_timing": {"method": "a start and a stop HIP event bound to every dispatch "
                                    "(hipExtLaunchKernel), over a second pass of the same "
                                    "steps; avg_launch_us is the dispatch's end minus its "
                                    "begin timestamp, the span a rocprofv3 kernel trace "
                                    "reports",
                          "empty_kernel_us": round(empty_us, 3),
                          "ms_per_step_with_events": round(ms_prof, 5)},
        "kernels": kernels,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(spec, off, idx, W, G, psw, args.cpu_sample_lookups,
                                           torch)
    tb.close()
    print(json.dumps(res))


if __name__ == "__main__":
    main()
