#!/usr/bin/env python3
"""TBE forward + backward (row-wise Adagrad) throughput on one MI355X.

One step = tbe_forward + tbe_backward_rowwise_adagrad (which runs the whole
preprocessing: transposition, radix sort, run-length encoding, classification)
over one batch of the workload; inputs are resident in HBM before timing.
Default workload: the large configuration (64 tables x 5M rows x 128 fp16,
B = 65536, L ~ Poisson(32)+1, Zipf 1.1, int32: 138 M lookups), the largest
that fits one GPU.

Timing: W warm-up steps, then K timed steps, each preceded (outside its
timing) by a 1 GiB scratch write that evicts the last-level cache, so every
step starts cold; HIP events around the forward and the backward of every
step give the per-step split.  Then, untimed for the headline: the same
steps back to back (warm), the fused long-run path, the preprocessing moved
into the forward (tbe_forward_preprocess + backward on the preprocessed
workspace, as the pages report it: forward, backward, sum), and a pass with
a start and a stop event bound to every kernel dispatch for per-kernel times.

Prints one JSON line: lookups/s (the headline), the roofline of the dominant
kernel on algorithmic bytes (each stream and unique row once: the step's
compulsory traffic), step-level byte fractions, per-kernel
figures, and the single-threaded CPU oracle timed on a bounded sample of the
same workload (whole tables, one pinned core).

Other modes: --calibrate-copy (a plain 1 GiB device copy, for counter
calibration), --pmc-summary DIR (turn rocprofv3 --pmc CSV output into the
committed counter summary).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
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
    "validate_check": "validate.hip", "validate_clear": "validate.hip",
    "dense_select": "bwd_dense.hip", "dense_partial": "bwd_dense.hip", "dense_update": "bwd.hip",
}
# kernels whose source includes the exact counts x grad_out product
COUNT_MMA_KERNELS = ("dense_partial", "bwd_hist_partial")
# rocprofv3 kernel names -> the library's kernel families (tbe_prof_read names)
KERNEL_FAMILIES = (
    ("fwd_bal_kernel", "fwd_pool"), ("fwd_pool_kernel", "fwd_pool"),
    ("fwd_hist_kernel", "fwd_hist"), ("tile_map_kernel", "tile_map"),
    ("transpose_scatter_kernel", "transpose"),
    ("radix_upsweep", "radix_upsweep"), ("first_upsweep", "radix_upsweep"),
    ("radix_scan", "radix_scan"),
    ("sort_pass_kernel", "radix_downsweep"), ("rle_kernel", "rle"),
    ("classify_kernel", "classify"), ("chunk_order_kernel", "chunk_order"),
    ("bwd_single_kernel", "bwd_single"), ("bwd_tiny_kernel", "bwd_tiny"),
    ("bwd_medium_kernel", "bwd_medium"), ("bwd_chunk_fused_kernel", "bwd_chunk_fused"),
    ("bwd_chunk_kernel", "bwd_chunk"), ("bwd_long_update_kernel", "bwd_long_update"),
    ("bwd_hist_partial_kernel", "bwd_hist_partial"),
    ("bwd_hist_count_kernel", "bwd_hist_partial"), ("bwd_hist_weighted_kernel", "bwd_hist_partial"),
    ("bwd_hist_update_kernel", "bwd_hist_update"),
    ("dense_select_kernel", "dense_select"), ("dense_partial_kernel", "dense_partial"),
    ("dense_update_kernel", "dense_update"),
    ("validate_clear_kernel", "validate_clear"), ("validate_offsets_kernel", "validate_check"),
    ("validate_indices_kernel", "validate_check"), ("validate_clamp_kernel", "validate_repair"),
)
COLD_FLUSH_BYTES = 1 << 30


def kernel_family(name):
    """The library's kernel family of a profiler kernel name (None for others)."""
    m = re.search(r"(\w+)\s*[<(]", name.replace("(anonymous namespace)", ""))
    base = m.group(1) if m else name
    return next((v for k, v in KERNEL_FAMILIES if base == k), None)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="C5", choices=["C1", "C2", "C3", "C4", "C5"])
    ap.add_argument("--fused", action="store_true",
                    help="headline step with the fused long-run countdown path")
    ap.add_argument("--validate", action="store_true",
                    help="run tbe_validate (check only) at the start of every step")
    ap.add_argument("--checked", action="store_true",
                    help="forward with the input checks fused in (tbe_forward_checked)")
    ap.add_argument("--bwd-hist", action="store_true",
                    help="histogram-reuse backward (one small table: C4), no preprocessing")
    ap.add_argument("--hist-reuse", action="store_true",
                    help="with --bwd-hist: the forward saves its row counts "
                         "(tbe_forward_preprocess, TBE_FWD_SAVE_HIST) and the backward reads "
                         "them instead of the indices")
    ap.add_argument("--schedule", default="serial", choices=["overlap", "fork", "auto", "serial"],
                    help="headline schedule. overlap: tbe_forward_preprocess (preprocessing on "
                         "a side stream during the forward), then the backward on the "
                         "preprocessed workspace; fork: the backward's run classes on three "
                         "streams; auto: fork below 64 Mi lookups; serial: one stream")
    ap.add_argument("--warm", action="store_true",
                    help="no cache flush between timed steps (headline on warm caches)")
    ap.add_argument("--quick", action="store_true",
                    help="skip the secondary passes (warm, fused, overlap split)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-lookups", type=int, default=8_000_000,
                    help="cap on lookups in the CPU oracle sample (whole tables)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--pmc-summary", metavar="DIR",
                    help="summarize rocprofv3 --pmc CSV files under DIR (no GPU work)")
    ap.add_argument("--pmc-workload", default=None, help="workload key of --pmc-summary")
    ap.add_argument("--pmc-out", default=os.path.join(ROOT, "profiles", "pmc_traffic.json"))
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
# the hot-row contraction of the long runs: batches without per-sample
# weights from this many lookups on, at most this many rows per table
DENSE_MIN_LOOKUPS = 8 << 20
DENSE_ROWS = 128


def dense_applies(spec, N):
    return (not spec.weighted and N >= DENSE_MIN_LOOKUPS and spec.T <= 128
            and any(d % 16 == 0 and d <= 256 for d in spec.dims))


def workload_stats(spec, off, idx):
    """Per-table lookups, unique rows, the run-length classes the backward
    splits runs into, and the long runs the contraction takes (the smallest
    threshold of at least max(256, B/256) that at most 128 runs reach, on
    tables with D a multiple of 16 up to 256) (host, from the inputs)."""
    B = spec.B
    dense = dense_applies(spec, int(off[-1]))
    st = []
    for t in range(spec.T):
        lo, hi = int(off[t * B]), int(off[(t + 1) * B])
        _, cnt = np.unique(idx[lo:hi], return_counts=True)
        s = dict(n=hi - lo, U=int(cnt.size), D=spec.dims[t], mean=spec.pooling[t] == 1,
                 max_sl=int(cnt.max(initial=0)))
        for name, a, b in SL_CLASSES:
            m = (cnt >= a) if b is None else ((cnt >= a) & (cnt < b))
            s["n_" + name] = int(m.sum())
            s["N_" + name] = int(cnt[m].sum())
        s["chunks"] = int(((cnt[cnt >= 256] + 255) // 256).sum())
        s["n_hot"] = s["N_hot"] = 0
        if dense and spec.dims[t] % 16 == 0 and spec.dims[t] <= 256:
            lens = cnt[cnt >= 256]
            thr = max(256, min(B // 256, 1 << 30))
            if int((lens >= thr).sum()) > DENSE_ROWS:
                thr = int(np.sort(lens)[::-1][DENSE_ROWS]) + 1
            hot = lens[lens >= thr]
            s["n_hot"], s["N_hot"] = int(hot.size), int(hot.sum())
        st.append(s)
    return st


def byte_model(spec, st):
    """Algorithmic bytes per kernel family and step (unit: one lookup; s_i index bytes, s_w weight bytes,
    psi = 1 with per-sample weights):
      forward   compulsory N(s_i + 4psi) + (TB+1)s_i + sum_t U_t D_t s_w + B Dtot 4
                logical    the same with N_t D_t s_w in place of U_t D_t s_w
      backward  compulsory N(s_i + 16 + 8psi) + (TB+1)s_i + sum_t U_t(2 D_t s_w + 8 + 16)
                           + B Dtot 4
                logical    the same with N_t 4 D_t in place of B Dtot 4
    The backward's terms are attributed to the kernels that make those
    accesses in a one-pass design: the transposition reads the indices (and
    weights) and offsets and writes key and bag (8N); the run-length pass
    reads the keys (4N) and writes run starts and keys (8U); the
    classification reads those (8U); each update kernel reads the bag (and
    weight) of its lookups (4 + 4psi per lookup), its share of grad_out once
    (compulsory) or one row per lookup (logical), and reads and writes each of
    its rows and momenta once.  The radix passes and the chunk order add
    nothing to the model (a one-pass grouping would not make them), so they
    count as pure overhead against it."""
    si = 4 if spec.itype == "i32" else 8
    sw = 4 if spec.wdtype == "f32" else 2
    psi = 1 if spec.weighted else 0
    T, B = spec.T, spec.B
    N = sum(s["n"] for s in st)
    U = sum(s["U"] for s in st)
    G_bytes = out_bytes = B * spec.dtot * 4
    comp, logi = {}, {}
    off_b = (T * B + 1) * si
    comp["fwd_pool"] = (N * (si + 4 * psi) + off_b + out_bytes
                        + sum(s["U"] * s["D"] * sw for s in st))
    logi["fwd_pool"] = (N * (si + 4 * psi) + off_b + out_bytes
                        + sum(s["n"] * s["D"] * sw for s in st))
    if T == 1:
        E, D = spec.rows[0], spec.dims[0]
        comp["fwd_hist"] = N * si + (B + 1) * si + E * D * sw + B * D * 4
        logi["fwd_hist"] = logi["fwd_pool"]
    comp["transpose"] = N * (si + 4 * psi) + off_b + 8 * N
    for k in ("tile_map", "radix_upsweep", "radix_scan", "radix_downsweep", "chunk_order"):
        comp[k] = 0
    comp["rle"] = 4 * N + 8 * U
    comp["classify"] = 8 * U
    for k in list(comp):
        logi.setdefault(k, comp[k])
    kern = {"single": "bwd_single", "tiny": "bwd_tiny", "medium": "bwd_medium",
            "long": "bwd_chunk", "hot": "dense_partial"}
    for k in ("bwd_single", "bwd_tiny", "bwd_medium", "bwd_chunk", "bwd_long_update",
              "dense_partial", "dense_update", "dense_select"):
        comp[k] = logi[k] = 0
    for s in st:
        D = s["D"]
        rmw = 2 * D * sw + 8  # weight row and momentum, read and written once
        for cls, k in kern.items():
            lk, runs = s["N_" + cls], s["n_" + cls]
            if cls == "long":  # the hot long runs are the contraction's
                lk, runs = lk - s["N_hot"], runs - s["n_hot"]
            per_lookup = lk * (4 + 4 * psi)
            comp[k] += per_lookup + G_bytes * lk / max(N, 1)
            logi[k] += per_lookup + lk * 4 * D
            upd = runs * rmw
            tgt = {"long": "bwd_long_update", "hot": "dense_update"}.get(cls, k)
            comp[tgt] += upd
            logi[tgt] += upd
    comp["bwd_chunk_fused"] = comp["bwd_chunk"] + comp["bwd_long_update"]
    logi["bwd_chunk_fused"] = logi["bwd_chunk"] + logi["bwd_long_update"]
    if T == 1:  # histogram-reuse backward: the contraction reads indices, offsets and G once
        D = spec.dims[0]
        comp["bwd_hist_partial"] = N * (si + 4 * psi) + (B + 1) * si + B * D * 4
        comp["bwd_hist_update"] = sum(s["U"] * (2 * s["D"] * sw + 8) for s in st)
        logi["bwd_hist_partial"] = comp["bwd_hist_partial"]
        logi["bwd_hist_update"] = comp["bwd_hist_update"]
    comp["validate_clear"] = logi["validate_clear"] = 16
    comp["validate_check"] = logi["validate_check"] = N * si + off_b
    totals = dict(
        fwd_comp=comp["fwd_pool"],
        bwd_comp=N * (si + 16 + 8 * psi) + off_b + G_bytes
        + sum(s["U"] * (2 * s["D"] * sw + 24) for s in st),
        fwd_logi=logi["fwd_pool"],
        bwd_logi=N * (si + 16 + 8 * psi) + off_b + sum(s["n"] * 4 * s["D"] for s in st)
        + sum(s["U"] * (2 * s["D"] * sw + 24) for s in st))
    return comp, logi, totals


def source_hash(kernel):
    f = KERNEL_SOURCES.get(kernel, "prep.hip")
    d = os.path.join(ROOT, "table_embedding_amd", "csrc")
    h = hashlib.sha256()
    names = (f, "tbe_common.h") + (("count_mma.h",) if kernel in COUNT_MMA_KERNELS else ())
    for name in names:  # the kernel's file and the shared device helpers
        h.update(open(os.path.join(d, name), "rb").read())
    return h.hexdigest()[:16]


def counter_entry(kernel, workload):
    """The committed rocprofv3 counter summary of a kernel family, if it was
    taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        e = json.load(open(p))[workload][kernel]
    except (KeyError, ValueError):
        return None
    if e.get("source_sha256_16") != source_hash(kernel):
        return None
    return e


# ---------------------------------------------------------------- CPU leg

def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec, off, idx, W_dev, G_dev, psw_dev, cap, torch):
    """The oracle (single-threaded C, one pinned core) on whole tables of the
    same workload: forward, then backward with its preprocessing."""
    import oracle
    B = spec.B
    tables, n = [], 0
    for t in range(spec.T):
        nt = int(off[(t + 1) * B] - off[t * B])
        if tables and n + nt > cap:
            break
        tables.append(t)
        n += nt
    sub = tables
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
        return (w.numpy().copy() if spec.wdtype == "f32"
                else w.view(torch.int16).numpy().view(np.uint16).copy())

    W = [host(W_dev[t]) for t in sub]
    M = [np.zeros(spec.rows[t], np.float32) for t in sub]
    oracle.build(force=False)
    cores_total = os.cpu_count()
    prev = os.sched_getaffinity(0)
    core = min(prev)
    os.sched_setaffinity(0, {core})
    try:
        t0 = time.perf_counter()
        oracle.forward(rows, dims, pooling, spec.wdtype, W, B, spec.itype, ix, o, psw)
        oracle.backward_rowwise_adagrad(rows, dims, pooling, spec.wdtype, W, M, B, spec.itype,
                                        ix, o, psw, G, spec.lr, spec.eps)
        dt = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, prev)
    return {"value": round((hi - lo) / dt, 1), "unit": "lookups/s", "cores": 1, "kind": "oracle",
            "sample": f"tables {sub[0]}..{sub[-1]} of {spec.T} ({hi - lo} lookups, all {B} bags "
                      f"of each), one forward + backward (with preprocessing) pass, {dt:.2f} s "
                      f"on 1 pinned core (core {core}) of {cores_total} host threads, "
                      f"{cpu_model()}",
            "seconds": round(dt, 3)}


# ------------------------------------------------------------- counters

def pmc_summary(args):
    """rocprofv3 --pmc CSV files (one run per counter set) -> bytes per launch
    per kernel family.  Read bytes: FETCH_SIZE, whose gfx950 expression counts
    every L2-to-fabric read request at its size (128 B via TCC_BUBBLE, 32 B via
    TCC_EA0_RDREQ_32B, 64 B the rest); write bytes: WRITE_SIZE (64 B and 32 B
    requests).  Each is scaled by the factor that makes a plain 1 GiB device
    copy (--calibrate-copy, profiled the same way: the runtime's copyBuffer
    kernel) read and write 1 GiB.  TCC_HIT / TCC_MISS, when present,
    give the L2 hit rate."""
    import csv
    rows = []
    for f in glob.glob(os.path.join(args.pmc_summary, "**", "*counter_collection.csv"),
                       recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    acc = {}  # (kernel name, dispatch id) -> {counter: value}
    for r in rows:
        name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
        key = (name, r.get("Dispatch_Id"), r.get("Correlation_Id"))
        # per-instance values (NAME[i]) and _sum reductions add up to one total
        cn = re.sub(r"\[\d+\]$", "", r["Counter_Name"])
        cn = cn[:-4] if cn.endswith("_sum") else cn
        acc.setdefault(key, {})[cn] = acc.get(key, {}).get(cn, 0.0) + float(r["Counter_Value"])

    def read_b(c):  # FETCH_SIZE is already request-size-resolved on gfx950 (32/64/128 B)
        return 1024 * c["FETCH_SIZE"] if "FETCH_SIZE" in c else None

    def write_b(c):
        return 1024 * c["WRITE_SIZE"] if "WRITE_SIZE" in c else None

    fam = {}
    cal = {"read": [], "write": []}
    for (name, _, _), c in acc.items():
        r, w = read_b(c), write_b(c)
        if "copyBuffer" in name:  # the runtime's blit copy of --calibrate-copy
            if r is not None:
                cal["read"].append(r)
            if w is not None:
                cal["write"].append(w)
            continue
        f = kernel_family(name)
        if f is None:
            continue
        e = fam.setdefault(f, {"read": [], "write": [], "hit": [], "miss": []})
        if r is not None:
            e["read"].append(r)
        if w is not None:
            e["write"].append(w)
        if "TCC_HIT" in c:
            e["hit"].append(c["TCC_HIT"])
        if "TCC_MISS" in c:
            e["miss"].append(c["TCC_MISS"])
    rs = (1 << 30) / np.median(cal["read"]) if cal["read"] else 1.0
    ws = (1 << 30) / np.median(cal["write"]) if cal["write"] else 1.0
    out = json.load(open(args.pmc_out)) if os.path.exists(args.pmc_out) else {}
    wk = out.setdefault(args.pmc_workload, {})
    for f, e in sorted(fam.items()):
        if not e["read"] or not e["write"]:
            continue
        rd, wr = rs * float(np.mean(e["read"])), ws * float(np.mean(e["write"]))
        ent = {"bytes_per_launch": int(rd + wr), "read_bytes": int(rd), "write_bytes": int(wr),
               "read_scale": round(rs, 4), "write_scale": round(ws, 4),
               "source_sha256_16": source_hash(f)}
        if e["hit"] and e["miss"]:
            h, m = float(np.mean(e["hit"])), float(np.mean(e["miss"]))
            ent["l2_hit_rate"] = round(h / max(h + m, 1.0), 4)
        wk[f] = ent
    json.dump(out, open(args.pmc_out, "w"), indent=1, sort_keys=True)
    print(json.dumps({"workload": args.pmc_workload, "read_scale": rs, "write_scale": ws,
                      "kernels": wk}, indent=1))


# -------------------------------------------------------------------- main

def calibrate_copy(torch):
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    print(json.dumps({"calibration_copy_bytes": n, "launches": 13,
                      "copy_gbs": round(2 * n / (ms * 1e6), 1)}))


def pct(a, q):
    return float(np.percentile(np.asarray(a, np.float64), q))


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args)
        return
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
    B = spec.B
    tb = te.TBE(spec.rows, spec.dims, spec.pooling, W, M)
    ws = tb.workspace(B, N)
    out = torch.empty((B, spec.dtot), dtype=torch.float32, device="cuda")
    base = (te.TBE_BWD_FUSED_LONG if args.fused else 0) | (te.TBE_BWD_HIST if args.bwd_hist else 0)
    conc = {"serial": 0, "overlap": 0, "auto": te.TBE_BWD_CONCURRENT_AUTO}.get(
        args.schedule, te.TBE_BWD_CONCURRENT)
    err = torch.zeros(te.TBE_VALIDATE_WORDS, dtype=torch.int32, device="cuda")
    flush_buf = torch.empty(COLD_FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    err_u = torch.zeros(te.TBE_VALIDATE_WORDS, dtype=torch.uint32, device="cuda")
    reuse = args.bwd_hist and args.hist_reuse

    def fwd(overlap):
        if args.validate:
            te.tbe_validate(tb.plan, B, d_idx, d_off, N, err)
        if reuse:
            tb.forward_and_preprocess(B, d_idx, d_off, psw, out, flags=te.TBE_FWD_SAVE_HIST)
        elif overlap:
            tb.forward_and_preprocess(B, d_idx, d_off, psw, out)
        elif args.checked:
            te.tbe_forward_checked(tb.plan, B, d_idx, d_off, N, psw, out, err_u)
        else:
            te.tbe_forward(tb.plan, B, d_idx, d_off, N, psw, out)

    def bwd(flags, overlap):
        f = flags | (te.TBE_BWD_PREPROCESSED if (overlap or reuse) else 0)
        te.tbe_backward_rowwise_adagrad(tb.plan, B, d_idx, d_off, N, psw, G, spec.lr, spec.eps,
                                        ws, f)

    def run(steps, flags, overlap, cold, wall=False):
        """`steps` steps, each with events around its forward and backward;
        cold: a 1 GiB scratch write before each step, outside its events."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            if cold:
                flush_buf.fill_(float(i))
            ev[i][0].record()
            fwd(overlap)
            ev[i][1].record()
            bwd(flags, overlap)
            ev[i][2].record()
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t0
        f = [e[0].elapsed_time(e[1]) for e in ev]
        b = [e[1].elapsed_time(e[2]) for e in ev]
        tot = [x + y for x, y in zip(f, b)]
        r = {"mean_ms": float(np.mean(tot)), "median_ms": pct(tot, 50), "p10_ms": pct(tot, 10),
             "p90_ms": pct(tot, 90), "fwd_ms": float(np.median(f)), "bwd_ms": float(np.median(b))}
        if wall:
            r["wall_s"] = wall_s
        return r

    overlap = args.schedule == "overlap"
    flags = base | conc
    run(args.warmup, flags, overlap, cold=False)
    print(f"[bench] warmup done ({args.warmup} steps), timing {args.steps}", file=sys.stderr,
          flush=True)
    head = run(args.steps, flags, overlap, cold=not args.warm, wall=True)
    ms = head["mean_ms"]
    secondary = {}
    if not args.quick:
        print("[bench] secondary passes", file=sys.stderr, flush=True)
        secondary["warm_back_to_back"] = run(args.steps, flags, overlap, cold=False)
        if not args.bwd_hist:
            secondary["serial_two_launch"] = run(args.steps, 0, False, cold=True)
            secondary["serial_fused"] = run(args.steps, te.TBE_BWD_FUSED_LONG, False, cold=True)
            secondary["preprocess_in_forward"] = run(args.steps, 0, True, cold=True)

    # per-kernel durations: start/stop events bound to each dispatch, the same
    # steps as the headline (cold), untimed for the headline
    te.tbe_prof_enable(True)
    prof_pass = run(args.steps, flags, overlap, cold=not args.warm)
    prof = te.tbe_prof_read()
    te.tbe_prof_calibrate(200)
    torch.cuda.synchronize()
    n_e, t_e = te.tbe_prof_read()["empty"]
    empty_us = 1000 * t_e / n_e
    te.tbe_prof_enable(False)

    st = workload_stats(spec, off, idx)
    comp, logi, tot = byte_model(spec, st)
    kernels = {}
    for k, (n, total_ms) in prof.items():
        kern_us = max(1000 * total_ms / n, 1e-3)
        per_step_ms = kern_us * n / args.steps / 1000
        ent = counter_entry(k, args.config + ("_hist" if args.bwd_hist else ""))
        kernels[k] = {"launches_per_step": n / args.steps, "ms_per_step": round(per_step_ms, 5),
                      "avg_launch_us": round(kern_us, 3),
                      "algorithmic_bytes_per_step": int(comp.get(k, 0)),
                      "frac_of_peak_algorithmic": round(
                          comp.get(k, 0) / (per_step_ms * 1e6) / HBM_PEAK_GBS, 4),
                      "counter_bytes_per_launch": None if ent is None else ent["bytes_per_launch"],
                      "l2_hit_rate": None if ent is None else ent.get("l2_hit_rate")}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom]
    bytes_per_launch = comp.get(dom, 0) / dk["launches_per_step"]
    achieved = bytes_per_launch / (dk["avg_launch_us"] * 1e3)  # GB/s
    if "fwd_hist" in kernels:  # the histogram forward's own model (counts x table)
        tot["fwd_comp"] = tot["fwd_logi"] = comp["fwd_hist"]
    if args.bwd_hist:
        tot["bwd_comp"] = tot["bwd_logi"] = comp["bwd_hist_partial"] + comp["bwd_hist_update"]
    step_comp = tot["fwd_comp"] + tot["bwd_comp"]
    step_logi = tot["fwd_logi"] + tot["bwd_logi"]
    per_kernel_counter = {k: kernels[k]["counter_bytes_per_launch"] for k in kernels}
    step_counter = (sum(v * kernels[k]["launches_per_step"] for k, v in per_kernel_counter.items())
                    if kernels and all(v is not None for v in per_kernel_counter.values())
                    else None)
    lookups_s = N / (ms / 1e3)
    n_runs = sum(s["U"] for s in st)
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
                   "lookups": N, "tables": spec.T, "bags_per_table": B,
                   "unique_rows": n_runs, "hottest_run": max(s["max_sl"] for s in st),
                   "index_type": spec.itype, "long_run_path": "fused" if args.fused else
                   "two-launch", "schedule": args.schedule,
                   "cache": "warm" if args.warm else "cold (1 GiB scratch write before each step)",
                   "backward": ("histogram contraction on the forward's saved counts" if reuse
                                else "histogram contraction" if args.bwd_hist
                                else "run pipeline"),
                   "input_validation": ("separate pass (tbe_validate)" if args.validate
                                        else "fused into the forward (tbe_forward_checked)"
                                        if args.checked else "off")},
        "timing": {"mean_ms": round(head["mean_ms"], 5), "median_ms": round(head["median_ms"], 5),
                   "p10_ms": round(head["p10_ms"], 5), "p90_ms": round(head["p90_ms"], 5),
                   "fwd_ms": round(head["fwd_ms"], 5), "bwd_ms": round(head["bwd_ms"], 5),
                   "wall_s_timed_loop": round(head["wall_s"], 4),
                   "note": "HIP events around each step's forward and backward; ms_per_step is "
                           "their mean over the timed steps"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": dk["counter_bytes_per_launch"],
                     "bytes_model": "algorithmic: each stream and unique row once"},
        "hbm": {"algorithmic_bytes_per_step": int(step_comp),
                "algorithmic_gbs": round(step_comp / (ms * 1e6), 1),
                "frac_of_peak_algorithmic": round(step_comp / (ms * 1e6) / HBM_PEAK_GBS, 4),
                "logical_bytes_per_step": int(step_logi),
                "effective_gbs_logical": round(step_logi / (ms * 1e6), 1),
                "counter_bytes_per_step": None if step_counter is None else int(step_counter),
                "counter_gbs": None if step_counter is None else
                round(step_counter / (ms * 1e6), 1),
                "counter_frac_of_peak": None if step_counter is None else
                round(step_counter / (ms * 1e6) / HBM_PEAK_GBS, 4),
                "traffic_ratio": None if step_counter is None or not step_comp else
                round(step_counter / step_comp, 3),
                "counter_source": "profiles/pmc_traffic.json: rocprofv3 L2-to-fabric (EA) read and "
                                  "write bytes per launch (request-size-resolved, calibrated on "
                                  "a 1 GiB copy); these include last-level-cache (MALL) hits, so "
                                  "they bound HBM traffic from above"},
        "secondary": {k: {kk: round(vv, 5) for kk, vv in v.items()} for k, v in
                      secondary.items()},
        "kernel_timing": {"method": "a start and a stop HIP event bound to every dispatch "
                                    "(hipExtLaunchKernel), over a pass of the same (cold) steps "
                                    "after the timed one; avg_launch_us is the dispatch's end "
                                    "minus its begin timestamp, the span a rocprofv3 kernel trace "
                                    "reports",
                          "empty_kernel_us": round(empty_us, 3),
                          "ms_per_step_with_events": round(prof_pass["mean_ms"], 5)},
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
