"""Throughput of the batched weighted L2 isotonic fit on one MI355X.

One step = one iso_fit_ex call (all stages of the fit) over the 1 x 10^8 fp32 mixed row
(y_i = sin(8 pi i/n) + 2 i/n + N(0, 0.05^2), w ~ LogUniform[0.1, 10]), inputs resident in HBM.
Prints one JSON line: elements/s of the whole fit, the roofline of the dominant kernel (its
algorithmic bytes over its average launch time, timed with HIP events inside the timed region),
the fit's whole-call fraction of the HBM roofline, rows/s on 65536 rows of 16 elements, the dense
1 x 10^8 fp64 nearly monotone row, and the CPU oracle timed on this host.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak


def _sync(torch):
    torch.cuda.synchronize()


def alg_bytes_per_elem(esz, weighted):
    """Algorithmic bytes of the fit per element: read y (+ w) and write z."""
    return esz * (3 if weighted else 2)


def stage_alg_bytes(stage, n_elems, esz, weighted):
    """Algorithmic bytes one launch of a stage's kernel moves: the row pass reads y (and w), the
    fit writes z; the scan, merge and ends kernels touch only workspace (no algorithmic bytes)."""
    if stage == "wave":
        return n_elems * esz * (2 if weighted else 1)
    if stage == "fit":
        return n_elems * esz
    return 0


def time_fit(torch, B, y, w, steps, warmup, rotate=None):
    """Times `steps` fits after `warmup`; `rotate` is a list of (y, w) input sets used in turn."""
    sets = rotate or [(y, w)]
    batch, n = sets[0][0].shape
    code = B.ISO_F64 if sets[0][0].dtype == torch.float64 else B.ISO_F32
    z = torch.empty_like(sets[0][0])
    ws, nbytes = B.workspace(batch, n, code, sets[0][1] is not None, sets[0][0].device)
    stream = B._stream(torch, sets[0][0].device)

    def call(k):
        yy, ww = sets[k % len(sets)]
        rc = B.iso_fit_ex(B._ptr(yy), B._ptr(ww), B._ptr(z), None, None, batch, n, code, B._ptr(ws), nbytes,
                          0, stream)
        if rc != 0:
            raise B.IsoError(rc, "iso_fit_ex")

    for k in range(warmup):
        call(k)
    _sync(torch)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for k in range(steps):
        call(k)
    ev1.record()
    _sync(torch)
    t1 = time.perf_counter()
    ms_events = ev0.elapsed_time(ev1) / steps
    ms_host = (t1 - t0) * 1e3 / steps
    # second pass of the same calls with per-stage events
    B.iso_prof_enable(1)
    for k in range(steps):
        call(k)
    _sync(torch)
    B.iso_prof_enable(0)
    st_ms, st_launch, calls = B.iso_prof_read()
    return z, ms_host, ms_events, st_ms, st_launch, calls


def roofline_of(stages_ms, stages_launch, calls, n_elems, esz, weighted):
    dom = max(stages_ms, key=lambda k: stages_ms[k])
    launches = max(stages_launch[dom], 1)
    avg_ms = stages_ms[dom] / launches
    per_launch_bytes = stage_alg_bytes(dom, n_elems, esz, weighted) * calls / launches
    achieved = per_launch_bytes / (avg_ms * 1e-3) / 1e9 if avg_ms > 0 else 0.0
    return {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "k_" + dom,
            "alg_bytes_per_launch": int(per_launch_bytes), "avg_launch_ms": round(avg_ms, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the short-row and dense-row lines")
    ap.add_argument("--only", choices=["mixed", "short", "dense"], default=None,
                    help="time one workload only (for profiler runs); implies --no-cpu")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (rows are independent and a "
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
    print("bench: generating mixed_1e8", file=sys.stderr, flush=True)
    y_h, w_h = W.mixed_1e8()
    n = y_h.shape[1]
    y = torch.from_numpy(y_h).to(dev)
    w = torch.from_numpy(w_h).to(dev)
    print("bench: timing mixed_1e8", file=sys.stderr, flush=True)
    z, ms_host, ms_ev, st_ms, st_la, calls = time_fit(torch, B, y, w, args.steps, args.warmup)
    esz = 4
    elems_per_s = n / (ms_host * 1e-3)
    fit_gbs = n * alg_bytes_per_elem(esz, True) / (ms_host * 1e-3) / 1e9
    roof = roofline_of(st_ms, st_la, calls, n, esz, True)
    stages = {k: round(v / max(calls, 1), 4) for k, v in st_ms.items()}

    out = {
        "metric": "elements/s and % HBM roofline: 1x10^8 row; rows/s at 65536x16",
        "value": round(elems_per_s, 1),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_host, 4),
        "ms_per_step_events": round(ms_ev, 4),
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
        "stage_ms": stages,
        "roofline": roof,
    }

    zo = None
    if not args.no_cpu:
        import oracle

        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        yd, wd = y_h.astype(np.float64), w_h.astype(np.float64)
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            zo = oracle.pav(yd, wd)
            times.append(time.perf_counter() - t0)
        t = sorted(times)[1]
        out["cpu_baseline"] = {"value": round(n / t, 1), "unit": "elements/s", "cores": 1, "kind": "oracle",
                               "sample": "the whole 1 x 10^8 row (fp64 pool adjacent violators, one thread), "
                                         "median of 3 runs of %.3f s" % t}
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
        _, msh, mse, sms, sla, sc = time_fit(torch, B, None, None, 200, 20, rotate=sets)
        out["short_rows_65536x16"] = {"rows_per_s": round(65536 / (msh * 1e-3), 1), "ms_per_call": round(msh, 5),
                                      "ms_per_call_events": round(mse, 5),
                                      "hbm_frac": round(65536 * 16 * 12 / (msh * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del sets, base_y, base_w
        torch.cuda.empty_cache()
        # dense row: 1 x 10^8 fp64 nearly monotone, unit weights passed explicitly
        print("bench: timing nearly_monotone_1e8 (fp64)", file=sys.stderr, flush=True)
        yd_h, wd_h = W.nearly_monotone_1e8()
        yd = torch.from_numpy(yd_h).to(dev)
        wd = torch.from_numpy(wd_h).to(dev)
        del yd_h, wd_h
        zd, msd, msde, dms, dla, dc = time_fit(torch, B, yd, wd, max(3, args.steps // 2), 2)
        nd = yd.shape[1]
        gbs = nd * alg_bytes_per_elem(8, True) / (msd * 1e-3) / 1e9
        # the exact fit of this row is y itself (every element its own block)
        dev_y = float(((zd - yd).abs() / (1 + yd.abs())).max().item())
        out["dense_1e8_f64"] = {"elements_per_s": round(nd / (msd * 1e-3), 1), "ms_per_call": round(msd, 4),
                                "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "achieved_gbs": round(gbs, 2),
                                "stage_ms": {k: round(v / max(dc, 1), 4) for k, v in dms.items()},
                                "roofline": roofline_of(dms, dla, dc, nd, 8, True),
                                "max_deviation_vs_y": dev_y}
    print(json.dumps(out), flush=True)


def run_only(args, torch, B, W, dev):
    """One workload, timed as in the full run; prints one JSON line of its own."""
    if args.only == "short":
        ys, wsh = W.short_rows_16()
        y, w = torch.from_numpy(ys).to(dev), torch.from_numpy(wsh).to(dev)
    elif args.only == "dense":
        yh, wh = W.nearly_monotone_1e8()
        y, w = torch.from_numpy(yh).to(dev), torch.from_numpy(wh).to(dev)
    else:
        yh, wh = W.mixed_1e8()
        y, w = torch.from_numpy(yh).to(dev), torch.from_numpy(wh).to(dev)
    print("bench: timing %s" % args.only, file=sys.stderr, flush=True)
    _, ms, mse, sms, sla, sc = time_fit(torch, B, y, w, args.steps, args.warmup)
    esz = y.element_size()
    n_el = y.numel()
    print(json.dumps({"workload": args.only, "ms_per_call": round(ms, 4), "ms_events": round(mse, 4),
                      "stage_ms": {k: round(v / max(sc, 1), 4) for k, v in sms.items()},
                      "hbm_frac": round(n_el * alg_bytes_per_elem(esz, True) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}),
          flush=True)


if __name__ == "__main__":
    main()
