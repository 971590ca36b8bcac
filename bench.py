#!/usr/bin/env python3
"""Benchmark of the error-bounded lossy compressor on one MI355X.

One step = compress + decompress of one synthetic batch (every stage of the
path: range reduction, quantization, duplicate-row detection, bit-plane
packing, stream assembly, and the inverse).  The default workload is 26 tables
x 8192 rows x 128 dims fp32, multi-hot pooled lookups, eb = 0.005 * range *
(1 + t/1000)^-1/2; ten batches (t = 0..9) are resident in HBM and steps cycle
through them, so the 1 GiB working set exceeds the 256 MiB Infinity Cache.

Prints ONE JSON line.  `value` is round-trip throughput in GB/s of
uncompressed input; the roofline object reports the dominant kernel's
algorithmic bytes per launch over its HIP-event-measured duration.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
WORKLOADS = {
    "c1": "1x2048x16 fp32 one-hot Zipf(1.05) lookups, abs eb 1e-4",
    "c2": "26x4096x64 fp32 one-hot Zipf lookups, eb 0.01*range",
    "c3": "26x8192x128 fp32 multi-hot pooled lookups, eb 0.005*range*(1+t/1000)^-1/2",
    "c4": "26x8192x128 fp32 gradients N(0,1e-3)+5% Laplace rows, sum-duplicated, abs eb 1e-5",
    "c5": "64x16384x256 fp32 one-hot Zipf(1.2) lookups, eb 0.01*range",
    "c5d40": "64x16384x256 fp32 one-hot Zipf-Mandelbrot(1.2, shift solved per table for "
             "an expected 40% repeated rows) lookups, eb 0.01*range",
}


HUFFMAN_SOURCES = ("ec_huffman.hip",)


def kernel_source_hash(coder: str = "bitpack") -> str:
    """Hash of the kernel sources a profile was taken on: the compressor's
    files, or the Huffman coder's file."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "error_bounded_lossy_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if (name in HUFFMAN_SOURCES) != (coder == "huffman"):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str, coder: str = "bitpack"):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(coder):
        return None
    return rec.get("hbm_bytes_per_launch")


def _host_cpus():
    """(usable host CPUs, CPU model string)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def _oracle_cfg(w, tables):
    """Oracle configuration for a subset of the workload's tables (one
    segment each, P = 1: a table's segment depends on that table alone)."""
    import oracle as O
    T, B, D = w.shape
    return O.Config(T=len(tables), B=B, D=D, eb_mode=w.eb_mode,
                    eb=tuple(w.eb[t] for t in tables), sched_kind=w.sched_kind,
                    sched_t0=w.sched_t0)


def _oracle_segment_compress(job):
    """Worker of the all-cores leg: compress one table (one segment)."""
    import oracle as O
    cfg, it, x = job
    t0 = time.perf_counter()
    st = O.compress(cfg, it, x, debug=False).stream
    return st, time.perf_counter() - t0


def _oracle_segment_decompress(job):
    import oracle as O
    cfg, st = job
    t0 = time.perf_counter()
    O.decompress(cfg, st)
    return time.perf_counter() - t0


def cpu_baseline(w, min_seconds: float, workers: int):
    """The oracle (single-threaded C, as it stands) on bounded samples of one
    batch of the workload, run before the GPU is touched (the all-cores leg
    forks worker processes):
      - one core: round trips of two tables at a time until min_seconds of
        CPU work, compress and decompress timed separately;
      - all cores: one oracle per segment (table) in a pool of `workers`
        processes, the batch's tables repeated until about min_seconds/2 of
        wall time, compress then decompress."""
    import multiprocessing as mp
    import numpy as np
    import oracle as O
    O.build(force=False)
    x = w.x.numpy()
    T, B, D = x.shape
    nbytes_t = 4 * B * D
    n_cpu, model = _host_cpus()
    tc = td = 0.0
    done = tables = 0
    t = 0
    while tc + td < min_seconds:
        sel = [t % T, (t + 1) % T]
        xs = np.ascontiguousarray(x[sel])
        cfg = _oracle_cfg(w, sel)
        t0 = time.perf_counter()
        c = O.compress(cfg, w.iteration, xs, debug=False)
        t1 = time.perf_counter()
        O.decompress(cfg, c.stream)
        t2 = time.perf_counter()
        tc += t1 - t0
        td += t2 - t1
        done += xs.nbytes
        tables += 2
        t += 2
    one = {"value": round(done / (tc + td) / 1e9, 5), "unit": "GB/s", "cores": 1,
           "kind": "oracle",
           "sample": f"{tables} table round trips ({tables}x{B}x{D} fp32, "
                     f"{done / 2**20:.0f} MiB) of batch t={w.iteration}, {tc + td:.1f} s",
           "compress_GBps": round(done / tc / 1e9, 5),
           "decompress_GBps": round(done / td / 1e9, 5),
           "host_cpus": n_cpu, "cpu_model": model}
    # all cores: enough repetitions of the batch's T segments for the target time
    per_seg = (tc + td) / tables
    reps = max(1, int(min_seconds / 2 * workers / (per_seg * T) + 0.5))
    jobs = [(_oracle_cfg(w, [tt]), w.iteration, np.ascontiguousarray(x[tt:tt + 1]))
            for _ in range(reps) for tt in range(T)]
    with mp.get_context("fork").Pool(workers) as pool:
        t0 = time.perf_counter()
        res = pool.map(_oracle_segment_compress, jobs, chunksize=1)
        t1 = time.perf_counter()
        pool.map(_oracle_segment_decompress, [(j[0], r[0]) for j, r in zip(jobs, res)],
                 chunksize=1)
        t2 = time.perf_counter()
    tot = len(jobs) * nbytes_t
    one["all_cores"] = {
        "value": round(tot / (t2 - t0) / 1e9, 5), "unit": "GB/s", "cores": workers,
        "compress_GBps": round(tot / (t1 - t0) / 1e9, 5),
        "decompress_GBps": round(tot / (t2 - t1) / 1e9, 5),
        "sample": f"{len(jobs)} segment round trips ({reps} x the {T} tables of batch "
                  f"t={w.iteration}, {tot / 2**20:.0f} MiB), one oracle per segment in "
                  f"{workers} processes, {t2 - t0:.1f} s wall"}
    return one


KERNEL_PREFIX = {"prep": "ec_prep", "encode": ("ec_encode", "ec_quantize"),
                 "assemble": ("ec_size", "ec_write"), "decode": ("ec_decode",)}
# the Huffman coder's two calls: encode (five kernels) and decode (two)
KERNEL_PREFIX_HUFF = {"huffman_encode": ("huff_clear", "huff_hist", "huff_book", "huff_size",
                                         "huff_write"),
                      "huffman_decode": ("huff_dec_book", "huff_decode")}


def dup_summary(batches):
    """Measured fraction of lookups that repeat an earlier row of their table,
    over the tables of the timed batches (one-hot workloads)."""
    d = [v for w in batches for v in w.dup]
    return {"mean": round(sum(d) / len(d), 4), "min": round(min(d), 4), "max": round(max(d), 4)}


def _short_kernel(name: str) -> str:
    name = name.replace("ec::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    return name.split("(")[0]


def _read_counter_csvs(d: str):
    """{kernel: {counter: [per-dispatch values]}} from a rocprofv3 --pmc run."""
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                k = _short_kernel(row.get("Kernel_Name", "?"))
                c = row.get("Counter_Name")
                out.setdefault(k, {}).setdefault(c, []).append(float(row.get("Counter_Value") or 0))
    return out


def summarize_counters(d: str, workload: str, copy_bytes: int, command: str,
                       coder: str = "bitpack"):
    """HBM traffic per launch of each pass of the path from four rocprofv3 --pmc
    runs (FETCH_SIZE and WRITE_SIZE of the workload, and of a plain copy of
    known size): each counter is scaled by bytes-moved / counter-reading of the
    copy; a pass of several kernels sums their per-dispatch averages.  Writes
    profiles/<pass>_<workload>_counters.json."""
    tag = f"huff_{workload}" if coder == "huffman" else workload
    wf = _read_counter_csvs(os.path.join(d, f"pmc_{tag}_fetch"))
    ww = _read_counter_csvs(os.path.join(d, f"pmc_{tag}_write"))
    cf = _read_counter_csvs(os.path.join(d, "pmc_copy_fetch"))
    cw = _read_counter_csvs(os.path.join(d, "pmc_copy_write"))

    def copy_kib(tab, counter):
        vals = [v for k, cs in tab.items() for v in cs.get(counter, [])]
        vals = sorted(vals)[len(vals) // 4:]  # drop warm-up outliers, keep the bulk
        return sum(vals) / len(vals)

    def mean(xs):
        return sum(xs) / len(xs)

    f_kib, w_kib = copy_kib(cf, "FETCH_SIZE"), copy_kib(cw, "WRITE_SIZE")
    f_scale = copy_bytes / (f_kib * 1024.0)
    w_scale = copy_bytes / (w_kib * 1024.0)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for kern, prefix in (KERNEL_PREFIX_HUFF if coder == "huffman" else KERNEL_PREFIX).items():
        names = sorted({k for k in list(wf) + list(ww) if k.startswith(prefix)})
        per = {}
        for nm in names:
            fk, wk = wf.get(nm, {}).get("FETCH_SIZE", []), ww.get(nm, {}).get("WRITE_SIZE", [])
            if fk and wk:
                per[nm] = {"dispatches": [len(fk), len(wk)], "fetch_kib": round(mean(fk), 1),
                           "write_kib": round(mean(wk), 1)}
        if not per:
            continue
        fetch = sum(v["fetch_kib"] for v in per.values())
        write = sum(v["write_kib"] for v in per.values())
        rec = {
            "pass": kern, "kernels": per, "workload": workload,
            "source_hash": kernel_source_hash(coder),
            "fetch_kib_per_launch": round(fetch, 1),
            "write_kib_per_launch": round(write, 1),
            "copy_calibration": {
                "kernel": "torch.neg over a float32 buffer (reads and writes copy_bytes each)",
                "copy_bytes": copy_bytes, "fetch_kib": round(f_kib, 1), "write_kib": round(w_kib, 1),
                "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5)},
            "hbm_fetch_bytes_per_launch": int(fetch * 1024 * f_scale),
            "hbm_write_bytes_per_launch": int(write * 1024 * w_scale),
            "hbm_bytes_per_launch": int(fetch * 1024 * f_scale + write * 1024 * w_scale),
            "command": command,
        }
        path = os.path.join(ROOT, "profiles", f"{kern}_{workload}_counters.json")
        with open(path, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        print(f"{path}: {rec['hbm_bytes_per_launch'] / 1e6:.2f} MB per launch "
              f"(fetch {fetch:.0f} KiB x {f_scale:.3f}, write {write:.0f} KiB x {w_scale:.3f})")


def summarize_stats(d: str, workload: str, command: str, coder: str = "bitpack",
                    stream_coder: str = "bitpack"):
    """Kernel-trace statistics (rocprofv3 --stats) of a bench run, as text:
    writes profiles/path_kernels_<workload>_kernel_stats.txt for the path
    kernels (path_kernels_<workload>_<stream coder>_... for a stream of
    Huffman or automatically chosen segments), or
    profiles/huffman_kernels_<workload>_kernel_stats.txt."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    what = "codes of " if coder == "huffman" else ""
    lines = [f"# rocprofv3 kernel statistics, workload {what}{workload}: {WORKLOADS[workload]}",
             f"# command: {command}",
             f"# source_hash: {kernel_source_hash(coder)}",
             f"{'kernel':<44} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}"]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    other = [0, 0.0, 0.0]
    for r in rows:
        name = _short_kernel(r["Name"])
        if not name.startswith(("huff_",) if coder == "huffman" else ("ec_", "huff_")):
            # synthetic-input generation and the like
            other[0] += int(r["Calls"])
            other[1] += float(r["TotalDurationNs"])
            other[2] += float(r["Percentage"])
            continue
        lines.append(f"{name[:44]:<44} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>9.2f} "
                     f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} "
                     f"{float(r['Percentage']):>6.2f}")
    lines.append(f"{'(all other kernels: input generation, torch)':<44} {other[0]:>6} "
                 f"{'':>9} {'':>9} {'':>9} {other[2]:>6.2f}")
    text = "\n".join(lines) + "\n"
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    stem = "huffman_kernels" if coder == "huffman" else "path_kernels"
    tag = workload if coder == "huffman" or stream_coder == "bitpack" else f"{workload}_{stream_coder}"
    path = os.path.join(ROOT, "profiles", f"{stem}_{tag}_kernel_stats.txt")
    with open(path, "w") as fh:
        fh.write(text)
    print(text, end="")


def copy_calibration(nbytes: int, reps: int):
    """A plain elementwise copy of known size for counter calibration."""
    import torch
    n = nbytes // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: {reps} x {nbytes} bytes", file=sys.stderr)


def workload_codes(w, torch):
    """Symbols q + 2047 of a workload batch: the quantization codes that the
    compressor itself computes for the batch (its debug hook writes them out
    while it compresses; an outlier's code is 0).  Input construction for the
    coder, outside any timed region."""
    import error_bounded_lossy_amd as ec
    T, B, D = w.shape
    sched = {"kind": w.sched_kind, "t0": w.sched_t0} if w.sched_kind else None
    plan = ec.Plan(T, B, D, 1, w.eb_mode, w.eb, schedule=sched, device=w.x.device)
    codes = torch.empty(T * B * D, dtype=torch.int32, device=w.x.device)
    plan.debug_attach(codes=codes)
    plan.compress(w.x, plan.empty_stream(), w.iteration)
    st = plan.ratio()[2]
    if st != ec.EC_OK:
        sys.exit(f"[bench] compressing the batch for its codes failed: {st}")
    return (codes + 2047).to(torch.int16)


def bench_huffman(args):
    """Canonical Huffman coder alone: one step = encode + decode of one
    batch's quantization codes (4 bytes of fp32 input per code), one codebook
    per table (the tables are the coder's segments)."""
    import torch
    import synth
    import error_bounded_lossy_amd as ec

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] codes of {args.batches} batches of {args.workload}", file=sys.stderr,
          flush=True)
    syms = [workload_codes(synth.workload(args.workload, iteration=i, device=dev), torch)
            for i in range(args.batches)]
    n = syms[0].numel()
    T = synth.SHAPES[args.workload][0]
    coder = ec.Huffman(dev, nseg=T)
    book, off, words = coder.buffers(n)
    out = torch.empty(n, dtype=torch.int16, device=dev)
    sizes = []
    for s in syms:  # compressed size of every batch (untimed)
        coder.encode(s, book, off, words)
        if coder.status() != ec.EC_OK:
            sys.exit("[bench] encode failed")
        nw = int(off[-1].item()) & 0xFFFFFFFF
        bk = book.view(T, ec.HUFF_BOOK_MAX)[:, :4].cpu().tolist()
        sizes.append(4 * nw + sum(ec.huff_book_bytes(b) for b in bk) + 4 * off.numel())

    def enc(i):
        coder.encode(syms[i % len(syms)], book, off, words)

    def dec():
        coder.decode(book, ec.HUFF_BOOK_MAX, off, words, n, out)

    for i in range(args.warmup):
        enc(i)
        dec()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 1)]
    e[0].record()
    for i in range(args.steps):
        enc(args.warmup + i)
        e[2 * i + 1].record()
        dec()
        e[2 * i + 2].record()
    torch.cuda.synchronize()
    t_enc = sum(e[2 * i].elapsed_time(e[2 * i + 1]) for i in range(args.steps))
    t_dec = sum(e[2 * i + 1].elapsed_time(e[2 * i + 2]) for i in range(args.steps))
    if coder.status() != ec.EC_OK:
        sys.exit("[bench] decode failed")
    last = syms[(args.warmup + args.steps - 1) % len(syms)]
    if not torch.equal(out, last):
        sys.exit("[bench] decoded codes differ from the input")
    ms = t_enc + t_dec
    step_s = ms / args.steps * 1e-3
    S = sum(sizes) / len(sizes)
    # decode call (codebook table + chunk decode): reads the stream, writes 2 B per code
    dec_s = t_dec / args.steps * 1e-3
    dec_bytes = S + 2 * n
    achieved = dec_bytes / dec_s / 1e9
    res = {
        "metric": "canonical Huffman encode+decode GB/s (fp32-equivalent: 4 B per code) per MI355X",
        "value": round(4 * n / step_s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic",
        "config": {"workload": f"codes of {args.workload}: {WORKLOADS[args.workload]}",
                   "codes": n, "codebooks": T, "batches_cycled": len(syms)},
        "encode_GBps": round(4 * n / (t_enc / args.steps * 1e-3) / 1e9, 2),
        "decode_GBps": round(4 * n / dec_s / 1e9, 2),
        "compression_ratio_vs_fp32": round(4 * n / S, 4),
        "bits_per_code": round(8 * S / n, 4),
        "roofline": {"bound": "hbm", "kernel": "decode call", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("huffman_decode", args.workload, "huffman"),
                     "algorithmic_bytes_per_launch": int(dec_bytes)},
    }
    print(json.dumps(res), flush=True)


def bench_window_sweep(args):
    """Table VI's experiment on the workload: the compression ratio of the
    stream with windowed references for W = 32, 64, 128, 255 (and the
    whole-segment references, W = 0), total bytes over the batches, each
    also relative to W = 32 as the table prints it; with each the warm
    compress and decompress rates."""
    import torch
    import synth
    import error_bounded_lossy_amd as ec

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    batches = [synth.workload(args.workload, iteration=i, device=dev) for i in range(args.batches)]
    w0 = batches[0]
    T, B, D = w0.shape
    N = T * B * D
    sched = {"kind": w0.sched_kind, "t0": w0.sched_t0} if w0.sched_kind else None
    rows = []
    for W in (32, 64, 128, 255, 0):
        print(f"[bench] window {W}", file=sys.stderr, flush=True)
        plan = ec.Plan(T, B, D, 1, w0.eb_mode, w0.eb, schedule=sched, device=dev, window=W)
        out = plan.empty_stream()
        y = torch.empty(T, B, D, dtype=torch.float32, device=dev)
        total = 0
        for w in batches:
            plan.compress(w.x, out, w.iteration)
            total += plan.ratio()[1]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for i in range(args.warmup):
            w = batches[i % len(batches)]
            plan.compress(w.x, out, w.iteration)
            plan.decompress(out, y)
        tc = td = 0.0
        for i in range(args.steps):
            w = batches[i % len(batches)]
            ev[0].record()
            plan.compress(w.x, out, w.iteration)
            ev[1].record()
            plan.decompress(out, y)
            ev[2].record()
            ev[2].synchronize()
            tc += ev[0].elapsed_time(ev[1])
            td += ev[1].elapsed_time(ev[2])
        if plan.ratio(raise_on_error=False)[-1] != ec.EC_OK:
            sys.exit("[bench] device error")
        rows.append({"window": W, "compression_ratio": round(4 * N * len(batches) / total, 4),
                     "compress_GBps": round(4 * N * args.steps / tc / 1e6, 1),
                     "decompress_GBps": round(4 * N * args.steps / td / 1e6, 1)})
        plan.close()
    base = rows[0]["compression_ratio"]
    for r in rows:
        r["ratio_vs_window_32"] = round(r["compression_ratio"] / base, 4)
    print(json.dumps({"experiment": "window sweep (Table VI)", "workload": args.workload,
                      "config": WORKLOADS[args.workload], "batches": len(batches),
                      "protocol": "warm, events around each call", "rows": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--batches", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="processes of the all-cores oracle leg (at most the usable CPUs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration)")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="write profiles/*_counters.json from rocprofv3 --pmc runs under DIR")
    ap.add_argument("--summarize-stats", metavar="DIR",
                    help="write profiles/*_kernel_stats.txt from a rocprofv3 --stats run under DIR")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    ap.add_argument("--coder", default="bitpack", choices=["bitpack", "huffman"],
                    help="huffman: time the standalone canonical Huffman coder on the "
                         "workload's codes")
    ap.add_argument("--stream-coder", default="bitpack", choices=["bitpack", "huffman", "auto"],
                    help="the segment coder of the compressed stream: bit planes, Huffman, "
                         "or per segment the smaller")
    ap.add_argument("--reuse-books", action="store_true",
                    help="Huffman segments keep their code across calls while it covers "
                         "their symbols (the batches cycled are successive iterations)")
    ap.add_argument("--window-sweep", action="store_true",
                    help="Table VI: the ratio of windowed references for W = 32 .. 255")
    args = ap.parse_args()
    if args.window_sweep:
        bench_window_sweep(args)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload,
                           args.copy_calibration or (256 << 20), args.command, args.coder)
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.workload, args.command, args.coder,
                        args.stream_coder)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 8)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported "
              f"(the library has no all-to-all across GPUs)", file=sys.stderr)
        sys.exit(2)

    if args.coder == "huffman":
        bench_huffman(args)
        return

    import torch
    import synth

    # the CPU baseline first: its worker processes fork before the GPU is used
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on a CPU sample", file=sys.stderr, flush=True)
        n_cpu, _ = _host_cpus()
        cpu = cpu_baseline(synth.workload(args.workload, iteration=0, device="cpu"),
                           args.cpu_seconds, min(n_cpu, args.cpu_workers))

    import error_bounded_lossy_amd as ec

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {args.batches} batches of {args.workload}", file=sys.stderr,
          flush=True)
    batches = [synth.workload(args.workload, iteration=i, device=dev) for i in range(args.batches)]
    w0 = batches[0]
    T, B, D = w0.shape
    N = T * B * D
    sched = {"kind": w0.sched_kind, "t0": w0.sched_t0} if w0.sched_kind else None
    coder = {"bitpack": ec.CODER_BITPACK, "huffman": ec.CODER_HUFFMAN,
             "auto": ec.CODER_AUTO}[args.stream_coder]
    plan = ec.Plan(T, B, D, 1, w0.eb_mode, w0.eb, schedule=sched, device=dev, coder=coder,
                   reuse_books=args.reuse_books)
    out = plan.empty_stream()
    y = torch.empty(T, B, D, dtype=torch.float32, device=dev)
    # read (untimed) before every timed call of the cold protocol: 512 MiB,
    # twice the Infinity Cache, so the call finds neither its input nor the
    # stream in any cache.  A read, not a write: a written buffer would leave
    # dirty lines whose write-back the next call would pay for.
    scratch = torch.ones(128 << 20, dtype=torch.int32, device=dev)

    def flush(i):
        torch.amax(scratch)

    # compressed size of every batch (untimed)
    crs, sizes = [], []
    for w in batches:
        plan.compress(w.x, out, w.iteration)
        cr, nb, _ = plan.ratio()
        crs.append(cr)
        sizes.append(nb)

    def batch(i):
        return batches[i % len(batches)]

    for i in range(args.warmup):
        w = batch(i)
        plan.compress(w.x, out, w.iteration)
        plan.decompress(out, y)
    torch.cuda.synchronize()

    # cold (primary): every call timed alone by events on its stream, after a
    # scratch write that evicts the caches
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4 * args.steps)]
    wall0 = time.perf_counter()
    for i in range(args.steps):
        w = batch(args.warmup + i)
        flush(i)
        ev[4 * i].record()
        plan.compress(w.x, out, w.iteration)
        ev[4 * i + 1].record()
        flush(i + 1)
        ev[4 * i + 2].record()
        plan.decompress(out, y)
        ev[4 * i + 3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    tc_ms = sum(ev[4 * i].elapsed_time(ev[4 * i + 1]) for i in range(args.steps))
    td_ms = sum(ev[4 * i + 2].elapsed_time(ev[4 * i + 3]) for i in range(args.steps))
    # the median step beside the mean (the value): compress + decompress per step
    step_ms = sorted(ev[4 * i].elapsed_time(ev[4 * i + 1]) + ev[4 * i + 2].elapsed_time(ev[4 * i + 3])
                     for i in range(args.steps))
    med_ms = (step_ms[(args.steps - 1) // 2] + step_ms[args.steps // 2]) / 2
    _, _, st = plan.ratio(raise_on_error=False)
    if st != 0:
        print(f"[bench] device status {st}", file=sys.stderr)
        sys.exit(1)

    # warm: the same steps back to back (the batches cycle through 1 GiB, so
    # each compression still reads its input from HBM; the stream it writes is
    # read by the decompression from the caches)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        w = batch(args.warmup + i)
        plan.compress(w.x, out, w.iteration)
        plan.decompress(out, y)
    e1.record()
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1)

    # per-kernel durations, cold protocol: every launch bracketed by HIP events
    # on the stream it runs on
    plan.profile_enable(True, max_launches=5 * args.steps + 8)
    for i in range(args.steps):
        w = batch(args.warmup + i)
        flush(i)
        plan.compress(w.x, out, w.iteration)
        flush(i + 1)
        plan.decompress(out, y)
    torch.cuda.synchronize()
    t_prep, n_prep = plan.profile_read(ec.KERNEL_PREP)
    t_enc, n_enc = plan.profile_read(ec.KERNEL_ENCODE)
    t_dec, n_dec = plan.profile_read(ec.KERNEL_DECODE)
    t_asm, n_asm = plan.profile_read(ec.KERNEL_ASSEMBLE)
    plan.profile_enable(False)
    _, _, st = plan.ratio(raise_on_error=False)
    if st != 0:
        print(f"[bench] device status {st}", file=sys.stderr)
        sys.exit(1)

    rel = w0.eb_mode == ec.EB_REL_RANGE
    K = args.steps
    # compressed bytes: the batches the timed steps ran on, in total
    S_tot = sum(sizes[(args.warmup + i) % len(batches)] for i in range(K))
    S = S_tot / K
    tc = tc_ms / K * 1e-3
    td = td_ms / K * 1e-3
    step_s = tc + td
    # algorithmic bytes: compression reads x (twice with a range-relative
    # bound: the range pass, then quantization) and writes the stream;
    # decompression reads the stream and writes x^
    bytes_c = 4 * N * (2 if rel else 1) + S
    bytes_d = S + 4 * N
    # per launch: the input read by the range pass (REL; a range pass of its
    # own, or the range items inside the quantize launch for D = 64, 128) and
    # by the quantize pass, the stream written by assembly (by the one encode
    # kernel when there is no assembly pass), and both for decode
    enc_reads = 4 * N * (2 if rel and not n_prep else 1)
    kernels = {
        "encode": (t_enc / max(n_enc, 1), enc_reads + (0 if n_asm else S)),
        "decode": (t_dec / max(n_dec, 1), S + 4 * N),
    }
    if n_prep:
        kernels["prep"] = (t_prep / n_prep, 4 * N if rel else 0)
    if n_asm:
        kernels["assemble"] = (t_asm / n_asm, S)
    dom = max(kernels, key=lambda k: kernels[k][0])
    dom_ms, dom_bytes = kernels[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = load_traffic(dom, args.workload)
    warm_step = warm_ms / K * 1e-3
    res = {
        "metric": "compress+decompress GB/s (uncompressed) per MI355X; ratio at eb; % HBM roof",
        "value": round(4 * N / step_s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "median": {"ms_per_step": round(med_ms, 5), "value": round(4 * N / (med_ms * 1e-3) / 1e9, 2)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOADS[args.workload]}", "tables": T,
                   "batch": B, "dim": D, "chunks": 1, "batches_cycled": len(batches),
                   "stream_coder": args.stream_coder,
                   "reuse_books": bool(args.reuse_books),
                   "protocol": "cold: 512 MiB scratch read before each timed call",
                   **({"repeated_rows": dup_summary(batches)} if w0.dup else {})},
        "compress_GBps": round(4 * N / tc / 1e9, 2),
        "decompress_GBps": round(4 * N / td / 1e9, 2),
        "compression_ratio": round(4 * N * K / S_tot, 4),
        "compression_ratio_per_batch": [round(c, 4) for c in crs],
        "hbm_roof_frac_roundtrip": round((bytes_c + bytes_d) / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "hbm_roof_frac_compress": round(bytes_c / tc / 1e9 / HBM_PEAK_GBS, 4),
        "hbm_roof_frac_decompress": round(bytes_d / td / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": {"compress": int(bytes_c), "decompress": int(bytes_d)},
        "warm": {"value": round(4 * N / warm_step / 1e9, 2), "ms_per_step": round(warm_ms / K, 5),
                 "hbm_roof_frac_roundtrip":
                     round((bytes_c + bytes_d) / warm_step / 1e9 / HBM_PEAK_GBS, 4)},
        "kernel_ms": {k: round(v[0], 5) for k, v in kernels.items()},
        "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(dom_bytes)},
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
