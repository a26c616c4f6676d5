"""Throughput of the batched weighted L2 isotonic fit on one MI355X.

One step = one iso_fit_ex call (every stage of the fit) over the 1 x 10^8 fp32 mixed row
(y_i = sin(8 pi i/n) + 2 i/n + N(0, 0.05^2), w ~ LogUniform[0.1, 10], seed 5), inputs resident
in HBM.  Prints one JSON line: elements/s of the whole fit; the roofline of the dominant kernel
(the fit's algorithmic bytes per element times the elements of one launch, over its average
launch time, timed with HIP events recorded on the launch stream inside the timed region) with
the HBM traffic measured by rocprofv3 counters when they were taken on the current kernel
sources; the fit's whole-call fraction of the HBM roofline; the backward; rows/s on 65536 rows of
16 elements; the 1 x 10^8 fp64 nearly monotone row (every chunk strictly increasing) and the same
row with a few reversals per chunk (the dense hull through the general chunk pass); the soft
rank; and the CPU oracle timed on this host.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]
    python bench.py --only mixed|dense|hull|calib|short|mono7|ramp|table1|vjp|vjpshort|softrank [--copy-calib]
    python bench.py --configs   (every measured configuration: per-call median and IQR, oracle)
    python bench.py --summarize-pmc WORKLOAD FETCH_DIR WRITE_DIR  (updates profiles/traffic.txt)

Algorithmic bytes per element are read y + read w + write z (sizeof(T) each).  Of these the
chunk pass (k_chunk) reads y and w; the fit (k_fit) writes z, except where the chunk pass already
wrote z = y (dense tiles).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")
COPY_BYTES = 1 << 30   # the calibration copy: 1 GiB read and 1 GiB written per launch
METRIC = "elements/s and % HBM roofline: 1x10^8 row; rows/s at 65536x16"


def source_hash():
    """sha256 of the HIP sources and headers the kernels are built from."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "weighted_isotonic_regression_amd", "csrc", "*")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")))
    for p in files:
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def alg_bytes_per_elem(esz, weighted):
    """Algorithmic bytes of the fit per element: read y (+ w) and write z."""
    return esz * (3 if weighted else 2)


CHUNK = 16384  # elements per chunk of a long row


def stage_alg_bytes(stage, n_elems, esz, weighted, whole_diagram):
    """Algorithmic bytes one call's kernels of a stage move (one row).

    whole_diagram: every full 16384-element chunk of the row is clean and strictly increasing
    (the nearly monotone row), so k_increasing reads y (and w) and writes z for all full chunks
    and the chunk pass and fit handle only the partial last chunk.  Otherwise k_increasing reads
    a 16-byte probe per lane of each full chunk, the chunk pass reads y (and w) and the fit writes
    z for the whole row.  The scan, merge and ends kernels touch only workspace."""
    full = (n_elems // CHUNK) * CHUNK if n_elems > 8192 else 0
    rest = n_elems - full if whole_diagram else n_elems
    reads = 2 if weighted else 1
    if stage == "increasing":
        return full * esz * (reads + 1) if whole_diagram else (full // CHUNK) * 64 * 16
    if stage == "chunk":
        return rest * esz * reads
    if stage == "fit":
        return rest * esz
    return 0


STAGE_KERNEL = {"increasing": "k_increasing", "chunk": "k_chunk", "exact": "k_chunk_exact", "scan": "k_scan",
                "merge": "k_merge_levels", "ends": "k_ends", "fit": "k_fit"}


def time_fit(torch, B, sets, steps, warmup, flags=0, stages=True):
    """Times `steps` fits after `warmup`; `sets` is a list of (y, w) input sets used in turn.
    With `stages`, per-stage HIP events are recorded on the launch stream inside the timed loop
    (their host-side cost is part of the time; calls of a few microseconds are timed without)."""
    batch, n = sets[0][0].shape
    code = B.ISO_F64 if sets[0][0].dtype == torch.float64 else B.ISO_F32
    z = torch.empty_like(sets[0][0])
    ws, nbytes = B.workspace(batch, n, code, sets[0][1] is not None, sets[0][0].device)
    stream = B._stream(torch, sets[0][0].device)

    def call(k):
        yy, ww = sets[k % len(sets)]
        rc = B.iso_fit_ex(B._ptr(yy), B._ptr(ww), B._ptr(z), None, None, batch, n, code, B._ptr(ws), nbytes,
                          flags, stream)
        if rc != 0:
            raise B.IsoError(rc, "iso_fit_ex")

    for k in range(warmup):
        call(k)
    torch.cuda.synchronize()
    B.iso_prof_read()  # forget anything recorded before
    B.iso_prof_enable(1 if stages else 0)
    t0 = time.perf_counter()
    for k in range(steps):
        call(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    B.iso_prof_enable(0)
    st_ms, st_launch, calls = B.iso_prof_read()
    ms_host = (t1 - t0) * 1e3 / steps
    return z, ms_host, st_ms, st_launch, calls


def time_vjp(torch, B, y, w, dev, steps):
    """iso_vjp on a row whose block starts come from one fit: reads g, y, w, z and the block starts
    and writes gy and gw (algorithmic bytes 6 sizeof(T) + 1 per element)."""
    print("bench: timing the backward", file=sys.stderr, flush=True)
    batch, n = y.shape
    code = B.ISO_F64 if y.dtype == torch.float64 else B.ISO_F32
    stream = B._stream(torch, dev)
    z = torch.empty_like(y)
    bs = torch.empty((batch, n), dtype=torch.uint8, device=dev)
    ws, nbytes = B.workspace(batch, n, code, True, dev)
    rc = B.iso_fit_ex(B._ptr(y), B._ptr(w), B._ptr(z), B._ptr(bs), None, batch, n, code, B._ptr(ws), nbytes,
                      0, stream)
    if rc != 0:
        raise B.IsoError(rc, "iso_fit_ex")
    del ws
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    g = torch.randn(y.shape, dtype=y.dtype, device=dev, generator=gen)
    gy, gw = torch.empty_like(y), torch.empty_like(y)

    def call():
        rc = B.iso_vjp(B._ptr(g), B._ptr(y), B._ptr(w), B._ptr(z), B._ptr(bs), B._ptr(gy), B._ptr(gw),
                       batch, n, code, stream)
        if rc != 0:
            raise B.IsoError(rc, "iso_vjp")

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    esz = y.element_size()
    nbytes_alg = batch * n * (6 * esz + 1)
    return {"elements_per_s": round(batch * n / (ms * 1e-3), 1), "ms_per_call": round(ms, 4),
            "alg_bytes": nbytes_alg, "hbm_frac": round(nbytes_alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def read_traffic():
    """{workload: {kernel: (fetch_bytes, write_bytes)}} from profiles/traffic.txt when it was
    measured on the current sources, else {}."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    out, sha = {}, None
    for line in open(TRAFFIC_FILE):
        line = line.strip()
        if line.startswith("source_sha256"):
            sha = line.split("=")[1].strip()
        elif line and not line.startswith("#") and "=" not in line:
            parts = line.split()
            if len(parts) >= 4:
                out.setdefault(parts[0], {})[parts[1]] = (float(parts[2]), float(parts[3]))
    return out if sha == source_hash() else {}


def roofline_of(workload, stages_ms, stages_launch, calls, n_elems, esz, weighted, whole_diagram, traffic):
    """The dominant stage's kernel against HBM: the fit's algorithmic bytes per element (read y,
    read w, write z) times the elements one launch processes, over its average launch time.
    `kernel_alg_bytes_per_launch` is what that kernel itself must move (its own reads and writes)."""
    dom = max(stages_ms, key=lambda k: stages_ms[k])
    launches = max(stages_launch[dom], 1)
    avg_ms = stages_ms[dom] / launches
    per_launch_bytes = alg_bytes_per_elem(esz, weighted) * n_elems * calls / launches
    own_bytes = stage_alg_bytes(dom, n_elems, esz, weighted, whole_diagram) * calls / launches
    achieved = per_launch_bytes / (avg_ms * 1e-3) / 1e9 if avg_ms > 0 else 0.0
    kern = STAGE_KERNEL[dom]
    t = traffic.get(workload, {}).get(kern)
    return {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None if t is None else int(t[0] + t[1]),
            "kernel": kern, "alg_bytes_per_launch": int(per_launch_bytes),
            "kernel_alg_bytes_per_launch": int(own_bytes), "avg_launch_ms": round(avg_ms, 4)}


def stage_line(st_ms, calls):
    return {k: round(v / max(calls, 1), 4) for k, v in st_ms.items()}


ONLY = {"mixed": "mixed_1e8", "dense": "nearly_monotone_1e8", "hull": "nearly_monotone_reversals_1e8",
        "short": "short_rows_16", "calib": "calibration",
        "mono7": "nearly_monotone_1e7", "ramp": "ramp_noise_4096", "table1": "noise_1e7_decreasing"}


def load_workload(torch, W, name, dev):
    yh, wh = W.WORKLOADS[ONLY[name]]()
    return yh, wh, torch.from_numpy(yh).to(dev), None if wh is None else torch.from_numpy(wh).to(dev)


# Every measured configuration: (name, generator, unit weights, decreasing, timed calls).  The
# unit-weight rows are run twice, with the weights passed as an array and with w = NULL.
CONFIGS = [
    ("cfg1_ramp_noise_4096_f64", "ramp_noise_4096", False, False, 200),
    ("cfg2_short_rows_65536x16_f32", "short_rows_16", True, False, 200),
    ("cfg3_calibration_512x131072_f32", "calibration", False, False, 20),
    ("cfg4_nearly_monotone_1e7_f64", "nearly_monotone_1e7", True, False, 20),
    ("cfg5_mixed_1e8_f32", "mixed_1e8", False, False, 10),
    ("gate_nearly_monotone_1e8_f64", "nearly_monotone_1e8", True, False, 10),
    ("table1_noise_1e7_f32_decreasing", "noise_1e7_decreasing", True, True, 20),
]
ROTATE_BYTES = 512 << 20  # written between timed calls of inputs smaller than this (the MALL is 256 MB)


def oracle_times(oracle, y, w, decreasing, threads):
    """The oracle on the same rows: one thread (median of 3 runs, of 200 for fits under 1 ms, or 1
    run when a run takes over 2 s; each through the oracle's Python binding),
    and, for batches, rows split across `threads` threads (the C oracle releases the GIL)."""
    import concurrent.futures

    import numpy as np

    yd = y.astype(np.float64)
    wd = None if w is None else w.astype(np.float64)
    times, z = [], None
    for k in range(200):
        t0 = time.perf_counter()
        z = oracle.pav(yd, wd, decreasing=decreasing)
        times.append(time.perf_counter() - t0)
        # three runs, or up to 200 for fits under a millisecond; one when a run takes over 2 s
        if times[-1] > 2.0 or (k >= 2 and times[-1] > 1e-3):
            break
    one = sorted(times)[len(times) // 2]
    multi = None
    if y.shape[0] > 1:
        parts = np.array_split(np.arange(y.shape[0]), threads)
        t0 = time.perf_counter()
        with concurrent.futures.ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda p: oracle.pav(yd[p], None if wd is None else wd[p], decreasing=decreasing), parts))
        multi = time.perf_counter() - t0
    return z, one, multi


def run_configs(args, torch, B, W, dev):
    """One JSON line per configuration: per-call GPU time (HIP events on the launch stream around
    each call; median and interquartile range), elements/s, rows/s, fraction of the HBM roofline,
    deviation from the oracle, and the oracle's own time on this host."""
    import numpy as np

    import oracle

    threads = max(1, min(16, os.cpu_count() or 1))
    host = {"cpu_count": os.cpu_count(), "oracle_threads": threads}
    try:
        with open("/proc/cpuinfo") as f:
            host["cpu_model"] = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    print(json.dumps({"host": host}), flush=True)
    stream = torch.cuda.current_stream(dev)
    scratch = torch.empty(ROTATE_BYTES, dtype=torch.uint8, device=dev)
    for name, gen, unit, dec, steps in CONFIGS:
        print("bench: config %s" % name, file=sys.stderr, flush=True)
        yh, wh = W.WORKLOADS[gen]()
        batch, n = yh.shape
        zo, t1, tm = oracle_times(oracle, yh, wh, dec, threads)
        y = torch.from_numpy(yh).to(dev)
        runs = [("passed", torch.from_numpy(wh).to(dev))] if wh is not None else []
        if unit:
            runs.append(("NULL", None))
        esz = y.element_size()
        code = B.ISO_F64 if esz == 8 else B.ISO_F32
        flags = B.ISO_FLAG_DECREASING if dec else 0
        rotate = y.numel() * esz * 3 < ROTATE_BYTES
        for wname, w in runs:
            z = torch.empty_like(y)
            ws, nbytes = B.workspace(batch, n, code, w is not None, dev)

            def call():
                rc = B.iso_fit_ex(B._ptr(y), B._ptr(w), B._ptr(z), None, None, batch, n, code, B._ptr(ws), nbytes,
                                  flags, B._stream(torch, dev))
                if rc != 0:
                    raise B.IsoError(rc, "iso_fit_ex")

            for _ in range(3):
                call()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            for k in range(steps):
                if rotate:
                    scratch.fill_(k & 255)
                ev[k][0].record(stream)
                call()
                ev[k][1].record(stream)
            torch.cuda.synchronize()
            ms = np.array([a.elapsed_time(b) for a, b in ev])
            med = float(np.median(ms))
            q1, q3 = (float(v) for v in np.percentile(ms, [25, 75]))
            alg = batch * n * alg_bytes_per_elem(esz, w is not None)
            zg = z.cpu().numpy().astype(np.float64)
            dev_o = float(np.max(np.abs(zg - zo) / (1 + np.abs(zo)))) if zg.size else 0.0
            line = {"config": name, "shape": [batch, n], "dtype": "f64" if esz == 8 else "f32", "weights": wname,
                    "direction": "decreasing" if dec else "increasing", "timed_calls": steps,
                    "rotated_inputs": rotate, "median_ms": round(med, 5), "iqr_ms": [round(q1, 5), round(q3, 5)],
                    "elements_per_s": round(batch * n / (med * 1e-3), 1), "rows_per_s": round(batch / (med * 1e-3), 1),
                    "alg_bytes": alg, "hbm_frac": round(alg / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "max_dev_vs_oracle": dev_o, "oracle_1thread_s": round(t1, 7),
                    "oracle_threads_s": None if tm is None else round(tm, 7)}
            print(json.dumps(line), flush=True)
            del z, ws
        del y, runs
        torch.cuda.empty_cache()


def run_only(args, torch, B, W, dev):
    """One workload, timed as in the full run; prints one JSON line of its own."""
    if args.copy_calib:
        # a plain device copy of known size, for scaling the memory counters
        a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        torch.cuda.empty_cache()
    if args.only == "softrank":
        print(json.dumps({"workload": "softrank", **time_soft_rank(torch, B, dev)}), flush=True)
        return
    if args.only in ("vjp", "vjpshort"):
        # the backward of the mixed 10^8 row, or of 65536 rows of 16 (rows of one tile)
        _, _, y, w = load_workload(torch, W, "mixed" if args.only == "vjp" else "short", dev)
        print(json.dumps({"workload": args.only, **time_vjp(torch, B, y, w, dev, args.steps)}), flush=True)
        return
    _, _, y, w = load_workload(torch, W, args.only, dev)
    print("bench: timing %s" % args.only, file=sys.stderr, flush=True)
    flags = B.ISO_FLAG_DECREASING if args.only == "table1" else 0
    _, ms, sms, sla, sc = time_fit(torch, B, [(y, w)], args.steps, args.warmup, flags=flags)
    esz = y.element_size()
    print(json.dumps({"workload": args.only, "ms_per_call": round(ms, 4), "stage_ms": stage_line(sms, sc),
                      "hbm_frac": round(y.numel() * alg_bytes_per_elem(esz, w is not None) / (ms * 1e-3) / 1e9 /
                                        HBM_PEAK_GBS, 4)}), flush=True)


def summarize_pmc(fetch_dir, write_dir):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of each kernel, scaled by the calibration copy's
    counters against its known 1 GiB read and 1 GiB write; writes profiles/traffic.txt."""
    def per_kernel(d, counter):
        acc = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                acc.setdefault(name, []).append(float(r["Counter_Value"]) * 1024.0)
        return acc

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    copy_f = [v for k, vs in fetch.items() if "elementwise" in k or "copy" in k.lower() for v in vs]
    copy_w = [v for k, vs in write.items() if "elementwise" in k or "copy" in k.lower() for v in vs]
    if not copy_f or not copy_w:
        raise SystemExit("no calibration copy kernel in the counter runs")
    sf = COPY_BYTES / (sorted(copy_f)[len(copy_f) // 2])
    sw = COPY_BYTES / (sorted(copy_w)[len(copy_w) // 2])
    def mine(k, key):
        if key in ("k_chunk", "k_chunk_exact"):
            # k_chunk<T, W, D, EXACT>: the first pass, or the exact pass over the chunks it left
            i = k.find("iso::k_chunk<")
            if i < 0:
                return False
            args = k[i + len("iso::k_chunk<"):].split(">")[0].split(",")
            return (args[-1].strip() == "true") == (key == "k_chunk_exact")
        return ("iso::%s<" % key) in k or ("iso::%s(" % key) in k

    # fit calls in the run: one k_chunk (long rows), k_row, k_wave (short rows) or k_tiny dispatch each
    calls = max(sum(len(vs) for k, vs in fetch.items() if mine(k, "k_chunk") or mine(k, "k_wave") or
                    mine(k, "k_row") or mine(k, "k_tiny")), 1)
    lines = []
    for key in ("k_tiny", "k_wave", "k_row", "k_increasing", "k_chunk", "k_chunk_exact", "k_scan_reduce", "k_scan_apply",
                "k_merge_levels", "k_ends", "k_fit"):
        fs = [v for k, vs in fetch.items() if mine(k, key) for v in vs]
        wsz = [v for k, vs in write.items() if mine(k, key) for v in vs]
        if fs and wsz:
            lines.append((key, sum(fs) / len(fs) * sf, sum(wsz) / len(wsz) * sw, len(fs) / calls))
    return sf, sw, lines


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the short-row and dense-row lines")
    ap.add_argument("--configs", action="store_true", help="measure every configuration, one JSON line each")
    ap.add_argument("--only", choices=sorted(ONLY) + ["vjp", "vjpshort", "softrank"], default=None,
                    help="time one workload only (for profiler runs)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="with --only: first run a 1 GiB device copy (memory-counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR"),
                    help="append the scaled counter traffic of a workload to profiles/traffic.txt")
    args = ap.parse_args()
    if args.summarize_pmc:
        wl, fd, wd = args.summarize_pmc
        sf, sw, lines = summarize_pmc(fd, wd)
        sha = source_hash()
        keep = []
        if os.path.exists(TRAFFIC_FILE):
            old = open(TRAFFIC_FILE).read().splitlines()
            if any(l.strip() == "source_sha256 = %s" % sha for l in old):
                keep = [l for l in old if l and not l.startswith("#") and "=" not in l and not l.startswith(wl + " ")]
        with open(TRAFFIC_FILE, "w") as f:
            f.write("# HBM bytes per launch of the fit's kernels: rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE\n")
            f.write("# (KiB per dispatch) scaled by the same counters for a 1 GiB device copy in the same run\n")
            f.write("# (latest scale factors: fetch %.4f, write %.4f).  Columns: workload kernel fetch_bytes\n"
                    % (sf, sw))
            f.write("# write_bytes launches_per_call.  Valid only for the kernel sources of this hash (bench.py\n")
            f.write("# checks it).\n")
            f.write("# Made by, for each workload W in mixed, dense, hull, short, calib, mono7\n")
            f.write("# (R = the repository root, OUT = an output directory, run from /tmp):\n")
            f.write("#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pf_W -o run -- \\\n")
            f.write("#     python3 $R/bench.py --only W --steps 2 --warmup 1 --copy-calib\n")
            f.write("#   (the same with WRITE_SIZE into pw_W), then\n")
            f.write("#   python bench.py --summarize-pmc NAME $OUT/pf_W $OUT/pw_W\n")
            f.write("# with NAME mixed_1e8_f32, dense_1e8_f64, hull_1e8_f64, short_65536x16_f32,\n")
            f.write("# calib_512x131072_f32, mono_1e7_f64 for those W.\n")
            f.write("source_sha256 = %s\n" % sha)
            for l in keep:
                f.write(l + "\n")
            for k, fb, wb, lpc in lines:
                f.write("%s %s %.0f %.0f %g\n" % (wl, k, fb, wb, lpc))
        print(open(TRAFFIC_FILE).read())
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (rows are independent and a "
              "long row is fitted on one device); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from weighted_isotonic_regression_amd import binding as B
    from weighted_isotonic_regression_amd import workloads as W

    B.load()
    dev = torch.device("cuda:0")
    if args.only:
        run_only(args, torch, B, W, dev)
        return
    if args.configs:
        run_configs(args, torch, B, W, dev)
        return
    traffic = read_traffic()
    print("bench: generating mixed_1e8", file=sys.stderr, flush=True)
    y_h, w_h, y, w = load_workload(torch, W, "mixed", dev)
    n = y_h.shape[1]
    print("bench: timing mixed_1e8", file=sys.stderr, flush=True)
    # The throughput is timed over whole calls; the per-stage HIP events (stage times and the dominant
    # kernel's launch duration) come from a second pass of the same number of calls, since each
    # event record adds to the call.
    z, ms_host, _, _, _ = time_fit(torch, B, [(y, w)], args.steps, args.warmup, stages=False)
    _, ms_staged, st_ms, st_la, calls = time_fit(torch, B, [(y, w)], args.steps, args.warmup)
    esz = 4
    elems_per_s = n / (ms_host * 1e-3)
    fit_gbs = n * alg_bytes_per_elem(esz, True) / (ms_host * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(elems_per_s, 1),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_host, 4),
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": "mixed_1e8: 1 x 10^8 fp32, y = sin(8 pi i/n) + 2 i/n + N(0, 0.05^2), "
                               "w ~ LogUniform[0.1, 10], seed 5",
                   "batch": 1, "n": n, "io_dtype": "f32", "weighted": True},
        "fit_hbm_roofline": {"alg_bytes": n * alg_bytes_per_elem(esz, True), "achieved": round(fit_gbs, 2),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(fit_gbs / HBM_PEAK_GBS, 4)},
        "stage_ms": stage_line(st_ms, calls),
        "ms_per_step_with_stage_events": round(ms_staged, 4),
        "roofline": roofline_of("mixed_1e8_f32", st_ms, st_la, calls, n, esz, True, False, traffic),
    }

    if not args.no_extra:
        out["backward_1e8_f32"] = time_vjp(torch, B, y, w, dev, max(3, args.steps // 2))

    if not args.no_cpu:
        import oracle

        # The oracle (one thread, fp64 pool adjacent violators) on the whole row, 20 runs (about
        # 12 s of CPU work).
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        yd, wd = y_h.astype(np.float64), w_h.astype(np.float64)
        times, zo = [], None
        for _ in range(20):
            t0 = time.perf_counter()
            zo = oracle.pav(yd, wd)
            times.append(time.perf_counter() - t0)
        t = sorted(times)[len(times) // 2]
        out["cpu_baseline"] = {"value": round(n / t, 1), "unit": "elements/s", "cores": 1, "kind": "oracle",
                               "sample": "the whole 1 x 10^8 mixed row, 20 runs of the fp64 pool-adjacent-"
                                         "violators oracle on one thread, median %.3f s (total %.1f s)"
                                         % (t, sum(times))}
        zg = z.cpu().numpy().astype(np.float64)
        out["max_deviation_vs_oracle"] = float(np.max(np.abs(zg - zo) / (1 + np.abs(zo))))
        del yd, wd, zo
    del y, w, z
    torch.cuda.empty_cache()

    if not args.no_extra:
        # 65536 rows of 16, fp32, unit weights passed explicitly; 64 rotated input sets (> 512 MB)
        print("bench: timing short_rows_16", file=sys.stderr, flush=True)
        ys, wsh = W.short_rows_16()
        base_y = torch.from_numpy(ys).to(dev)
        base_w = torch.from_numpy(wsh).to(dev)
        sets = [(base_y.roll(k, dims=0).contiguous(), base_w.clone()) for k in range(64)]
        _, msh, _, _, _ = time_fit(torch, B, sets, 200, 20, stages=False)
        out["short_rows_65536x16"] = {"rows_per_s": round(65536 / (msh * 1e-3), 1), "ms_per_call": round(msh, 5),
                                      "hbm_frac": round(65536 * 16 * 12 / (msh * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del sets, base_y, base_w
        torch.cuda.empty_cache()
        # dense row: 1 x 10^8 fp64 nearly monotone, unit weights passed explicitly
        print("bench: timing nearly_monotone_1e8 (fp64)", file=sys.stderr, flush=True)
        _, _, yd, wd = load_workload(torch, W, "dense", dev)
        zd, msd, _, _, _ = time_fit(torch, B, [(yd, wd)], max(3, args.steps // 2), 2, stages=False)
        _, _, dms, dla, dc = time_fit(torch, B, [(yd, wd)], max(3, args.steps // 2), 2)
        nd = yd.shape[1]
        gbs = nd * alg_bytes_per_elem(8, True) / (msd * 1e-3) / 1e9
        # the exact fit of this row is y itself (every element its own block)
        dev_y = float(((zd - yd).abs() / (1 + yd.abs())).max().item())
        out["dense_1e8_f64"] = {"elements_per_s": round(nd / (msd * 1e-3), 1), "ms_per_call": round(msd, 4),
                                "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "achieved_gbs": round(gbs, 2),
                                "stage_ms": stage_line(dms, dc),
                                "roofline": roofline_of("dense_1e8_f64", dms, dla, dc, nd, 8, True, True, traffic),
                                "max_deviation_vs_y": dev_y}
        del yd, wd, zd
        torch.cuda.empty_cache()
        # dense hull through the general chunk pass: the same row with a few reversals per chunk
        print("bench: timing nearly_monotone_reversals_1e8 (fp64)", file=sys.stderr, flush=True)
        _, _, yr, wr = load_workload(torch, W, "hull", dev)
        _, msr, _, _, _ = time_fit(torch, B, [(yr, wr)], max(3, args.steps // 2), 2, stages=False)
        _, _, rms, rla, rc = time_fit(torch, B, [(yr, wr)], max(3, args.steps // 2), 2)
        nr = yr.shape[1]
        gbs = nr * alg_bytes_per_elem(8, True) / (msr * 1e-3) / 1e9
        out["dense_hull_1e8_f64"] = {"elements_per_s": round(nr / (msr * 1e-3), 1), "ms_per_call": round(msr, 4),
                                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "achieved_gbs": round(gbs, 2),
                                     "stage_ms": stage_line(rms, rc),
                                     "roofline": roofline_of("hull_1e8_f64", rms, rla, rc, nr, 8, True, False,
                                                             traffic)}
        del yr, wr
        torch.cuda.empty_cache()
        out["soft_rank_f32"] = time_soft_rank(torch, B, dev)
    print(json.dumps(out), flush=True)


def time_soft_rank(torch, B, dev, reps=20):
    """The soft rank at the page's training-step shapes (Section 7.9, Table 6: standard normal
    values, eps = 1/n, fp32): median ms of the forward alone and of forward plus backward, each
    call bracketed by HIP events on the launch stream."""
    import numpy as np

    print("bench: timing the soft rank", file=sys.stderr, flush=True)
    res = {}
    stream = torch.cuda.current_stream(dev)
    for batch, n in ((256, 1000), (4, 100_000)):
        x = torch.from_numpy(np.random.default_rng(12).standard_normal((batch, n)).astype(np.float32)).to(dev)
        g = torch.from_numpy(np.random.default_rng(13).standard_normal((batch, n)).astype(np.float32)).to(dev)
        eps = 1.0 / n
        fwd, both = [], []
        for k in range(reps + 3):
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record(stream)
            r, perm, bs = B.soft_rank(x, eps)
            e1.record(stream)
            B.soft_rank_vjp(g, perm, bs, eps)
            e2.record(stream)
            torch.cuda.synchronize()
            if k >= 3:
                fwd.append(e0.elapsed_time(e1))
                both.append(e0.elapsed_time(e2))
        res["%dx%d" % (batch, n)] = {"eps": eps, "forward_ms": round(float(np.median(fwd)), 4),
                                     "forward_backward_ms": round(float(np.median(both)), 4)}
    return res


if __name__ == "__main__":
    main()
