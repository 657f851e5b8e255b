#!/usr/bin/env python3
"""Benchmark of the MRU hot path on one MI355X (gfx950).

One step = the whole path over one batch of seeded synthetic input already
resident in HBM: the forward prefix scan straight from the raw token vectors
(LDU build folded in: x -> P) and the backward scan (x, P, dL/dP -> dL/dM),
which rebuilds each input's factors the same way; the input state matrices are
never stored.  Prints ONE JSON line:

  value         tokens/s of the whole step (a token = one position of one batch
                row, all heads included), timed with HIP events over exactly
                --steps steps after --warmup untimed ones
  roofline      the dominant kernel's algorithmic bytes per launch / its average
                launch time (HIP events on the launch stream), against the
                8 TB/s HBM peak; `traffic` is the measured HBM bytes per launch
                from profiles/hbm_traffic.json when that record was taken on the
                current kernel sources, else null
  kernels       the same figures for every kernel of the step
  unfused       the separate kernels (build x -> M, scan M -> P, backward from M,
                and the build's own backward x, dM -> dx) timed alone, and the
                layer backward x, P, dL/dP -> dL/dx in one pass (bwd_dx)
  n16, n32      forward-scan throughput on the n=16 and n=32 workloads (from_x: the
                same scan from the raw token vectors, and build then scan)
  n16_fwd_bwd   forward and backward scans on the n=16 forward+backward workload,
                and its layer step from the raw token vectors (forward x -> P,
                one-pass backward to dL/dx) against the three-kernel backward
  small         the two small workloads (one 1024-token n=4 sequence; the 8x8x256
                n=8 step): launch-bound latencies
  next          the scaled forward, the orthogonal input builds and a
                token-by-token decode step with a carried state
  cpu_baseline  the fp64 oracle (oracle/) timed on the host on a bounded sample
                of the same workload, on one thread and split over worker
                processes; and the GPU step's outputs on the first batch rows
                checked against the oracle's (relative Frobenius error per
                matrix, with the 2e-4 / 5e-4 bounds)

Only one GPU is used: --gpus N with N > 1 exits with an explanation.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP32_PEAK_TFLOPS = 157.3
FP64_PEAK_TFLOPS = 78.6
METRIC = "MRU prefix-scan tokens/s + achieved HBM GB/s (frac of peak), n=8 and n=16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
# Untimed launches before each figure of the extra workloads.  Launched back to
# back, the n = 16 forward's time drifts before it settles, and again after the
# GPU has been idle (one box, launch by launch: 262 us, rising to 312 us by the
# tenth launch, back to 264 us by the fortieth; right after the compute-heavy
# forward from raw token vectors a steady 250-256 us): the clock and power
# management's transient, not the kernel's.  30 launches take the figures past
# most of it.
WARMUP_EXTRA = 30


# Counter records under profiles/, each workload's entry stamped with the hash of
# the library sources it was taken on (every .hip and .h of the package's csrc):
# a figure taken on other sources is not reported.
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_util.json")
# (grid, wave x token steps per dispatch) of the bench step's kernels
# (--summarize counters): C2L runs 8192 chains of 256 tokens, 8 chains per
# wave, 1024 waves of 64 lanes
COUNTER_STEPS = {"c2l": (1024 * 64, 1024 * 256)}
CSRC = os.path.join(ROOT, "matrix_prefix_product_amd", "csrc")
SIMDS = 1024          # 256 CUs x 4 SIMDs
XCDS = 8
NOMINAL_CLOCK_HZ = 2.4e9


def source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h"))):
        with open(os.path.join(CSRC, p), "rb") as f:
            h.update(p.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(kind: str, S: int, T: int, n: int) -> int:
    # Algorithmic bytes per matrix entry per token-head (4-byte entries), the
    # definition's own traffic: build reads x and writes M, forward reads M (or
    # x) and writes P, backward reads M (or x), P and dP and writes dM (or dx),
    # build backward reads x and dM and writes dx.
    per = {"build": 8, "fwd": 8, "bwd": 16, "fwd_x": 8, "bwd_x": 16, "build_bwd": 12,
           "bwd_dx": 16}[kind]
    return per * n * n * S * T


def design_bytes(kind: str, S: int, T: int, n: int) -> int:
    # The bytes a kernel moves by design, where that is less than the
    # algorithmic count: for n <= 8 the backwards from raw token vectors (bwd_x,
    # bwd_dx) read one stored prefix per 4 tokens and recompute the others, 13
    # bytes per entry instead of 16.
    if kind in ("bwd_x", "bwd_dx") and n <= 8:
        return 13 * n * n * S * T
    return algorithmic_bytes(kind, S, T, n)


def algorithmic_flops(kind: str, S: int, T: int, n: int) -> int:
    # serial-product flops: forward n^3 mult-adds per token-head, backward 2 n^3
    return {"build": n ** 3 // 3 * 2, "fwd": 2 * n ** 3, "bwd": 4 * n ** 3,
            "fwd_x": 2 * n ** 3, "bwd_x": 4 * n ** 3}[kind] * S * T


def _record(path: str, workload: str, kind: str):
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    w = rec.get("workloads", {}).get(workload)
    if not w or w.get("source_hash") != source_hash():
        return None
    return w.get("kernels", {}).get(kind)


def load_traffic(workload: str, kind: str):
    """Counted HBM bytes (read + written) per launch of this workload's kernel,
    when the record was taken on the current sources; else None."""
    k = _record(TRAFFIC_FILE, workload, kind)
    return None if not k else int(k["read_bytes"] + k["write_bytes"])


def load_mfma_util(workload: str, kind: str):
    """Matrix-core and vector-ALU busy fractions counted by rocprofv3 for this
    workload's kernel, when the record was taken on the current sources; else None."""
    return _record(MFMA_FILE, workload, kind)


# ---------------------------------------------------------------------------
# rocprofv3 summaries: `bench.py --summarize {trace,traffic,mfma} --profile-workload W
# DIR...` reads the CSV files rocprofv3 wrote under DIR (kernel_stats.csv of a
# --kernel-trace --stats run, counter_collection.csv of --pmc runs), prints the
# text summary kept under profiles/, and (traffic, mfma) updates the JSON record
# bench.py reports from.

def short_kernel(name: str) -> str:
    s = name.replace("void ", "").replace("mru::(anonymous namespace)::", "").replace("mru::", "")
    return re.sub(r"\(.*$", "", s).strip()


def kernel_kind(short: str):
    """The step a library kernel runs: build, fwd, fwd_x, bwd, bwd_x, bwd_dx,
    build_bwd (fwd*_scaled for the scaled forward), copy for the runtime's
    buffer copy; None for anything else."""
    if short.startswith("__amd_rocclr_copyBuffer"):
        return "copy"
    m = re.match(r"(\w+)<([^>]*)>", short)
    if not m:
        return None
    fam, args = m.group(1), [a.strip() for a in m.group(2).split(",")]
    # template arguments: fwd_*_kernel<n, ., ., FX, SC>, bwd_valu_kernel<n, R, TB, FX, DX>,
    # bwd_mfma_kernel<n, PF, FX, DX, KR>
    if fam in ("fwd_valu_kernel", "fwd_mfma_kernel"):
        return ("fwd_x" if args[3] == "true" else "fwd") + ("_scaled" if args[4] == "true" else "")
    if fam in ("bwd_valu_kernel", "bwd_mfma_kernel"):
        fx, dx = (args[3], args[4]) if fam == "bwd_valu_kernel" else (args[2], args[3])
        return "bwd_dx" if dx == "true" else ("bwd_x" if fx == "true" else "bwd")
    if fam in ("build_kernel", "build_mfma_kernel"):
        return "build"
    if fam in ("build_bwd_kernel", "build_bwd_mfma_kernel"):
        return "build_bwd"
    return None


def _csvs(dirs, suffix):
    out = []
    for d in dirs:
        for root, _, files in os.walk(d):
            out += [os.path.join(root, f) for f in files if f.endswith(suffix)]
    if not out:
        sys.exit(f"no *{suffix} under {dirs}")
    return sorted(out)


def read_counters(dirs):
    """{(kernel, grid): {"dur_ns": [...], counter: [per-dispatch values]}}"""
    import csv
    from collections import defaultdict
    per = defaultdict(lambda: defaultdict(dict))  # (kernel, grid) -> dispatch -> counter -> value
    dur = defaultdict(dict)
    for path in _csvs(dirs, "counter_collection.csv"):
        for r in csv.DictReader(open(path)):
            key = (short_kernel(r["Kernel_Name"]), int(r["Grid_Size"]))
            d = (path, r["Dispatch_Id"])
            c = per[key][d]
            c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            dur[key][d] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = {}
    for key, disp in per.items():
        rec = {"dur_ns": [dur[key][d] for d in disp]}
        for d, cs in disp.items():
            for c, v in cs.items():
                rec.setdefault(c, []).append(v)
        out[key] = rec
    return out


def _median(v):
    v = sorted(v)
    return v[len(v) // 2]


def summarize(what: str, dirs, workload: str, commands) -> None:
    head = [f"# {what} summary of the {workload} kernels, rocprofv3 on one MI355X",
            f"# library source hash {source_hash()}",
            "# commands (run from /tmp with TMPDIR=/tmp; REPO = repository root):"]
    head += [f"#   {c}" for c in commands]
    if what == "trace":
        import csv
        print("\n".join(head))
        print(f"{'kernel':56s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}")
        for path in _csvs(dirs, "kernel_stats.csv"):
            for r in csv.DictReader(open(path)):
                print(f"{short_kernel(r['Name'])[:56]:56s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                      f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f}")
        return
    data = read_counters(dirs)
    if what == "counters":
        # every counter of the runs, median per dispatch, and per wave and token
        # step (the dispatch's wave count x the workload's tokens per chain)
        sgrid, steps = COUNTER_STEPS.get(workload, (None, None))
        names = sorted({c for v in data.values() for c in v if c != "dur_ns"})
        head += [f"# median per dispatch; '/step' rows (kernels of grid {sgrid}) divide by waves x tokens "
                 f"per chain = {steps} (the {workload} step kernels, one chunk per chain)" if steps else
                 "# median per dispatch"]
        print("\n".join(head))
        print(f"{'kernel':48s} {'grid':>9s} {'us':>9s} " + " ".join(f"{c:>22s}" for c in names))
        for (k, grid), v in sorted(data.items(), key=lambda kv: -_median(kv[1]["dur_ns"])):
            if not all(c in v for c in names):
                continue
            vals = " ".join(f"{_median(v[c]):22.0f}" for c in names)
            print(f"{k[:48]:48s} {grid:9d} {_median(v['dur_ns']) / 1e3:9.1f} {vals}")
            if steps and grid == sgrid:
                print(f"{'  /step':48s} {'':9s} {'':9s} " + " ".join(f"{_median(v[c]) / steps:22.2f}" for c in names))
        return
    path = TRAFFIC_FILE if what == "traffic" else MFMA_FILE
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        rec = {}
    kernels = {}
    if what == "traffic":
        # scale: the runtime's copy of a known size (1 GiB read + 1 GiB written) in
        # the same runs; without one, the factors of the record's last copy
        cal = rec.get("copy_kernel")
        for (k, grid), v in data.items():
            # the 1 GiB copy of copy_reference (other runtime copies are small)
            if kernel_kind(k) == "copy" and "FETCH_SIZE" in v and "WRITE_SIZE" in v \
                    and abs(_median(v["WRITE_SIZE"]) - 2 ** 20) < 0.05 * 2 ** 20:
                f, w = _median(v["FETCH_SIZE"]), _median(v["WRITE_SIZE"])
                cal = {"name": f"{k} (torch copy_ of 1 GiB)", "bytes_read": 2 ** 30, "bytes_written": 2 ** 30,
                       "FETCH_SIZE_KiB": f, "WRITE_SIZE_KiB": w,
                       "fetch_scale": round(2 ** 30 / (f * 1024), 3), "write_scale": round(2 ** 30 / (w * 1024), 3)}
        if cal is None:
            sys.exit("no copy kernel in these runs and no earlier scale on record")
        rec["copy_kernel"] = cal
        rec["counters"] = "rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (KiB per dispatch, median)"
        head += [f"# scale: {cal['name']} reads FETCH_SIZE {cal['FETCH_SIZE_KiB']:.1f} KiB and WRITE_SIZE "
                 f"{cal['WRITE_SIZE_KiB']:.1f} KiB per 1 GiB,",
                 f"#   so read bytes = {cal['fetch_scale']} x FETCH_SIZE x 1024 and write bytes = "
                 f"{cal['write_scale']} x WRITE_SIZE x 1024"]
        cols = f"{'kernel':48s} {'grid':>9s} {'us':>9s} {'FETCH_KiB':>12s} {'WRITE_KiB':>12s} {'read_bytes':>13s} {'write_bytes':>13s}"
        lines = []
        for (k, grid), v in sorted(data.items(), key=lambda kv: -_median(kv[1]["dur_ns"])):
            if "FETCH_SIZE" not in v or "WRITE_SIZE" not in v:
                continue
            f, w = _median(v["FETCH_SIZE"]), _median(v["WRITE_SIZE"])
            rb, wb = int(cal["fetch_scale"] * f * 1024), int(cal["write_scale"] * w * 1024)
            lines.append(f"{k[:48]:48s} {grid:9d} {_median(v['dur_ns']) / 1e3:9.1f} {f:12.1f} {w:12.1f} {rb:13d} {wb:13d}")
            kind = kernel_kind(k)
            if kind and kind != "copy":
                kernels[kind] = {"kernel": k, "grid": grid, "FETCH_SIZE_KiB": f, "WRITE_SIZE_KiB": w,
                                 "read_bytes": rb, "write_bytes": wb}
    else:
        # matrix-core busy: SQ_VALU_MFMA_BUSY_CYCLES (summed over the SIMDs; an
        # f64 16x16x4 product counts 64 cycles, an f32 one 32) over the SIMD-cycles
        # of the kernel, with GRBM_GUI_ACTIVE (summed over the 8 XCDs) as the
        # kernel's cycles; vector ALU: SQ_INSTS_VALU wave instructions at 4 issue
        # cycles each (wave64 on a 16-lane SIMD) over the same SIMD-cycles
        head += ["# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs)",
                 "#   (the counter sums SIMD-cycles: 64 per f64 16x16x4 product, 32 per f32 one; the n = 16",
                 "#   build reads exactly 4 x 64 per token);",
                 "# valu_busy = 4 x SQ_INSTS_VALU / (GRBM_GUI_ACTIVE / 8 x 1024) (4 issue cycles per wave64",
                 "#   instruction); the *_clk figures take the kernel's duration x 2.4 GHz as its cycles;",
                 "# clock_GHz = GRBM_GUI_ACTIVE / 8 / duration; medians over the dispatches"]
        cols = (f"{'kernel':48s} {'grid':>9s} {'us':>9s} {'mfma_busy':>10s} {'mfma_clk':>9s} {'valu_busy':>10s} "
                f"{'valu_clk':>9s} {'clock_GHz':>9s} {'MFMA_BUSY':>14s} {'VALU_INSTS':>12s} {'GRBM_ACTIVE':>12s}")
        lines = []
        for (k, grid), v in sorted(data.items(), key=lambda kv: -_median(kv[1]["dur_ns"])):
            if "SQ_VALU_MFMA_BUSY_CYCLES" not in v or "GRBM_GUI_ACTIVE" not in v:
                continue
            mb, gr, us = _median(v["SQ_VALU_MFMA_BUSY_CYCLES"]), _median(v["GRBM_GUI_ACTIVE"]), _median(v["dur_ns"]) / 1e3
            vi = _median(v.get("SQ_INSTS_VALU", [0.0]))
            simd_cyc = gr / XCDS * SIMDS
            clk_cyc = us * 1e-6 * NOMINAL_CLOCK_HZ * SIMDS
            r = {"kernel": k, "grid": grid, "us": round(us, 1),
                 "mfma_busy": round(mb / simd_cyc, 4), "mfma_busy_clk": round(mb / clk_cyc, 4),
                 "valu_busy": round(4 * vi / simd_cyc, 4), "valu_busy_clk": round(4 * vi / clk_cyc, 4),
                 "clock_GHz": round(gr / XCDS / (us * 1e-6) / 1e9, 3),
                 "SQ_VALU_MFMA_BUSY_CYCLES": mb, "SQ_INSTS_VALU": vi, "GRBM_GUI_ACTIVE": gr}
            for c in ("SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F64", "SQ_INSTS_MFMA",
                      "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS"):
                if c in v:
                    r[c] = _median(v[c])
            lines.append(f"{k[:48]:48s} {grid:9d} {us:9.1f} {r['mfma_busy']:10.4f} {r['mfma_busy_clk']:9.4f} "
                         f"{r['valu_busy']:10.4f} {r['valu_busy_clk']:9.4f} {r['clock_GHz']:9.3f} {mb:14.0f} "
                         f"{vi:12.0f} {gr:12.0f}")
            kind = kernel_kind(k)
            if kind and kind != "copy":
                kernels[kind] = r
    rec.setdefault("workloads", {})[workload] = {"source_hash": source_hash(), "kernels": kernels,
                                                 "commands": list(commands)}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print("\n".join(head + [f"# machine-readable copy: profiles/{os.path.basename(path)}", cols] + lines))


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), read before the GPU is touched."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


# Batch rows of the timed workload whose GPU outputs the host leg checks
# against the oracle (all heads, all tokens).
PARITY_ROWS = 16
_POOL = {}  # inputs of the parallel oracle run, inherited by the forked workers


def _oracle_rows(bounds):
    """One worker's share of the parallel oracle run: batch rows [lo, hi)."""
    from threadpoolctl import threadpool_limits

    from oracle import build_ref, bwd_ref, scan_ref
    lo, hi = bounds
    x, R, n = _POOL["x"][lo:hi], _POOL["R"][lo:hi], _POOL["n"]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        M = build_ref(x, n)
        scan_ref(M)
        bwd_ref(M, R)
        return time.perf_counter() - t0


def cpu_leg(w, budget_s: float, max_workers: int = 16):
    """The fp64 oracle's build + forward + backward on the host, on a bounded
    sample of the workload (whole sequences, batch rows 0..nb-1, all heads):
    (i) in this process with BLAS on one thread, (ii) split over batch rows
    across forked worker processes, one thread each.  Runs before the GPU is
    touched (the workers are forked).  Returns the baseline record and the
    oracle's outputs for the first PARITY_ROWS batch rows."""
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import build_ref, bwd_ref, scan_ref
    from workloads import gen_R, gen_x

    T = min(w.T, 4096)

    def gen(rows):
        return (gen_x(w.B, w.H, T, w.n, w.sigma_off, w.sigma_diag, w.seed, b_idx=rows),
                gen_R(w.B, w.H, T, w.n, w.seed, b_idx=rows))

    def run(x, R):
        t0 = time.perf_counter()
        M = build_ref(x, w.n)
        P = scan_ref(M)
        dM = bwd_ref(M, R)
        return time.perf_counter() - t0, P, dM

    with threadpool_limits(limits=1):
        probe = min(w.B, 4)
        dt, _, _ = run(*gen(range(probe)))
        nb = int(min(w.B, max(probe, budget_s / max(dt / probe, 1e-9))))
        x, R = gen(range(nb))
        dt, P, dM = run(x, R)
    keep = min(nb, PARITY_ROWS)
    ref = (P[:keep].copy(), dM[:keep].copy())
    del P, dM

    workers = max(1, min(max_workers, len(os.sched_getaffinity(0)), nb))
    _POOL.update(x=x, R=R, n=w.n)
    cuts = [nb * k // workers for k in range(workers + 1)]
    with mp.get_context("fork").Pool(workers) as pool:
        pool.map(_oracle_rows, [(0, 1)] * workers)  # start every worker
        t0 = time.perf_counter()
        pool.map(_oracle_rows, list(zip(cuts[:-1], cuts[1:])))
        dt_par = time.perf_counter() - t0
    _POOL.clear()

    head_tokens = nb * w.H * T
    rec = {
        "value": head_tokens / w.H / dt,
        "unit": "tokens/s",
        "cores": 1,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{nb} batch rows x {w.H} heads x {T} tokens of {w.name} (fp64 numpy build_ref + "
                  f"scan_ref + bwd_ref, {dt:.1f} s, BLAS limited to 1 thread)",
        "head_tokens_per_s": head_tokens / dt,
        "parallel": {
            "value": head_tokens / w.H / dt_par,
            "unit": "tokens/s",
            "cores": workers,
            "cpu_model": cpu_model(),
            "sample": f"the same sample split over {workers} forked processes by batch rows, "
                      f"one BLAS thread each, {dt_par:.2f} s wall",
        },
    }
    return rec, ref


def cpu_parity(ref, gpu):
    """Relative Frobenius error per matrix of the GPU's P and dM rows against
    the oracle's (fp64 build from the same x), with the forward and backward
    bounds (2e-4, 5e-4)."""
    import numpy as np

    from oracle import rel_fro_err
    out = {"rows": f"batch rows 0..{ref[0].shape[0] - 1}, all heads and tokens"}
    for name, r, g, tol in (("P", ref[0], gpu[0], 2e-4), ("dM", ref[1], gpu[1], 5e-4)):
        e = rel_fro_err(g[: r.shape[0]].astype(np.float64), r)
        out[name] = {"max": float(e.max()), "median": float(np.median(e)),
                     "over_bound": int(np.sum(e > tol)), "bound": tol}
    return out


def kernel_record(kind, avg_ms, S, T, n, workload):
    b = algorithmic_bytes(kind, S, T, n)
    d = design_bytes(kind, S, T, n)
    gbs = b / (avg_ms * 1e-3) / 1e9
    traffic = load_traffic(workload, kind)
    return {
        "avg_us": round(avg_ms * 1e3, 2),
        "algorithmic_bytes": b,
        "achieved_GBs": round(gbs, 1),
        "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
        "design_bytes": d,
        "frac_hbm_design": round(d / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "frac_hbm_traffic": (None if traffic is None else
                             round(traffic / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)),
    }


def ws_ok(mpp, ws, B, H, T, n, direction):
    """The status word of the last scan on ws is 0 (plans with a workspace only);
    exits if a look-back wait timed out, since the timed outputs are invalid."""
    if mpp.workspace_bytes(B, H, T, n, direction) == 0:
        return True
    st = mpp.ws_status(ws)
    if st != 0:
        sys.exit(f"a look-back wait timed out (status {st}) on B={B} H={H} T={T} n={n}")
    return True


def fwd_only(mpp, torch, name, B, H, T, n, so, sd, reps, seed):
    """Forward scan alone on a large workload; inputs generated on the GPU from a seed."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    scale = torch.full((n, n), so, device="cuda")
    scale.fill_diagonal_(sd)
    x = (torch.randn((B, H, T, n, n), generator=g, device="cuda") * scale).reshape(B, H, T, n * n)
    x = x.contiguous()
    M = mpp.build_inputs(x, n)
    P = torch.empty_like(M)
    ws = torch.empty(max(mpp.workspace_bytes(B, H, T, n), 256), dtype=torch.uint8, device="cuda")

    def median_ms(fn):
        for _ in range(WARMUP_EXTRA):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        times = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
        return times[len(times) // 2]

    med = median_ms(lambda: mpp.scan_fwd(M, out=P, workspace=ws))
    ws_ok(mpp, ws, B, H, T, n, mpp.DIR_FWD)
    # the same scan from the raw token vectors (input matrices formed on chip), and
    # the two-call path it replaces, where that exists for this n
    from_x = None
    if n in mpp.FUSED_FWD_N:
        t_x = median_ms(lambda: mpp.scan_fwd_x(x, n, out=P, workspace=ws))
        ws_ok(mpp, ws, B, H, T, n, mpp.DIR_FWD)
        t_b = median_ms(lambda: mpp.build_inputs(x, n, out=M))
        from_x = {"median_us": round(t_x * 1e3, 1), "build_then_scan_us": round((t_b + med) * 1e3, 1),
                  "build_us": round(t_b * 1e3, 1),
                  "tokens_per_s": B * T / (t_x * 1e-3),
                  "matrix_util_counted": load_mfma_util(name, "fwd_x"),
                  "build_matrix_util_counted": load_mfma_util(name, "build")}
    del x
    S = B * H
    b = algorithmic_bytes("fwd", S, T, n)
    K, nch, Z, _ = mpp.scan_plan(B, H, T, n)
    # implementation MFMA/VALU work: one n^3 product per token, two for tokens in
    # chunks that need a carry (all but the first chunk of a sequence)
    prod = S * T * (2.0 if nch > 1 else 1.0) - (S * K if nch > 1 else 0)
    impl_flops = prod * 2 * n ** 3
    peak = FP64_PEAK_TFLOPS  # n = 16 and 32 keep an fp64 running state
    del M, P, ws
    torch.cuda.empty_cache()
    return {
        "workload": f"{name}: B={B},H={H},T={T},n={n}, forward scan only",
        "median_us": round(med * 1e3, 1),
        "tokens_per_s": B * T / (med * 1e-3),
        "achieved_GBs": round(b / (med * 1e-3) / 1e9, 1),
        "frac_hbm": round(b / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "plan": {"chunk": K, "chunks_per_seq": nch, "super": Z},
        "matrix_tflops": round(impl_flops / (med * 1e-3) / 1e12, 2),
        "matrix_peak_tflops": peak,
        "matrix_util": round(impl_flops / (med * 1e-3) / 1e12 / peak, 4),
        "matrix_util_counted": load_mfma_util(name, "fwd"),
        "from_x": from_x,
        "data": "synthetic, seeded on the GPU (torch.Generator), same scales as the workload",
    }


def fwd_bwd(mpp, torch, name, B, H, T, n, so, sd, reps, seed):
    """Forward and backward scans (M -> P, then M, P, dL/dP -> dL/dM) on the
    n = 16 forward+backward workload, and the layer step from the raw token
    vectors (x -> P, then x, P, dL/dP -> dL/dx in one pass) beside the
    three-kernel backward it replaces; inputs generated on the GPU from a seed,
    dL/dP drawn N(0, 1)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    scale = torch.full((n, n), so, device="cuda")
    scale.fill_diagonal_(sd)
    x = (torch.randn((B, H, T, n, n), generator=g, device="cuda") * scale).reshape(B, H, T, n * n)
    x_layer = x.contiguous()
    M = mpp.build_inputs(x_layer, n)
    del x
    R = torch.randn((B, H, T, n, n), generator=g, device="cuda")
    P = torch.empty_like(M)
    dM = torch.empty_like(M)
    ws_f = torch.empty(max(mpp.workspace_bytes(B, H, T, n, mpp.DIR_FWD), 256), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(max(mpp.workspace_bytes(B, H, T, n, mpp.DIR_BWD), 256), dtype=torch.uint8, device="cuda")
    t_f = _time(torch, lambda: mpp.scan_fwd(M, out=P, workspace=ws_f), reps)
    t_b = _time(torch, lambda: mpp.scan_bwd(M, P, R, out=dM, workspace=ws_b), reps)
    ws_ok(mpp, ws_f, B, H, T, n, mpp.DIR_FWD)
    ws_ok(mpp, ws_b, B, H, T, n, mpp.DIR_BWD)
    S = B * H
    out = {"workload": f"{name}: B={B},H={H},T={T},n={n}, forward scan then backward scan"}
    for kind, us in (("fwd", t_f), ("bwd", t_b)):
        K, nch, Z, _ = mpp.scan_plan(B, H, T, n, mpp.DIR_FWD if kind == "fwd" else mpp.DIR_BWD)
        # products per token: forward 1, backward 2 (state and dM); multi-chunk
        # plans run every token twice (aggregate, then from the carry), except
        # the forward's first chunk of each sequence
        per = 1 if kind == "fwd" else 2
        prod = per * S * T * (2.0 if nch > 1 else 1.0) - (S * K if kind == "fwd" and nch > 1 else 0)
        flops = prod * 2 * n ** 3
        b = algorithmic_bytes(kind, S, T, n)
        out[kind] = {
            "median_us": round(us, 1),
            "achieved_GBs": round(b / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "plan": {"chunk": K, "chunks_per_seq": nch, "super": Z},
            "matrix_tflops": round(flops / (us * 1e-6) / 1e12, 2),
            "matrix_peak_tflops": FP64_PEAK_TFLOPS,
            "matrix_util": round(flops / (us * 1e-6) / 1e12 / FP64_PEAK_TFLOPS, 4),
            "matrix_util_counted": load_mfma_util(name, kind),
        }
    out["tokens_per_s"] = B * T / ((t_f + t_b) * 1e-6)
    # the layer step from the raw token vectors: forward x -> P and the one-pass
    # backward x, P, dL/dP -> dL/dx, against the three-kernel backward it replaces
    # (build x -> M, backward to dL/dM, the build's gradient dL/dM -> dL/dx)
    x = x_layer
    dx = torch.empty_like(x)
    t_fx = _time(torch, lambda: mpp.scan_fwd_x(x, n, out=P, workspace=ws_f), reps)
    ws_ok(mpp, ws_f, B, H, T, n, mpp.DIR_FWD)
    t_dx = _time(torch, lambda: mpp.scan_bwd_dx(x, P, R, out=dx, workspace=ws_b), reps)
    ws_ok(mpp, ws_b, B, H, T, n, mpp.DIR_BWD)
    t_bx = _time(torch, lambda: mpp.scan_bwd_x(x, P, R, out=dM, workspace=ws_b), reps)
    t_build = _time(torch, lambda: mpp.build_inputs(x, n, out=M), reps)
    t_bm = _time(torch, lambda: mpp.scan_bwd(M, P, R, out=dM, workspace=ws_b), reps)
    t_bb = _time(torch, lambda: mpp.build_inputs_bwd(x, dM, out=dx), reps)
    out["layer_from_x"] = {
        "fwd_x_us": round(t_fx, 1),
        "bwd_dx_us": round(t_dx, 1),
        "step_us": round(t_fx + t_dx, 1),
        "step_tokens_per_s": B * T / ((t_fx + t_dx) * 1e-6),
        "bwd_x_us": round(t_bx, 1),
        "three_kernel_bwd_us": {"build": round(t_build, 1), "bwd": round(t_bm, 1),
                                "build_bwd": round(t_bb, 1), "total": round(t_build + t_bm + t_bb, 1)},
        "bwd_dx_algorithmic_GBs": round(algorithmic_bytes("bwd_dx", S, T, n) / (t_dx * 1e-6) / 1e9, 1),
        "bwd_dx_frac_hbm": round(algorithmic_bytes("bwd_dx", S, T, n) / (t_dx * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "matrix_util_counted": {"bwd_dx": load_mfma_util(name, "bwd_dx"), "bwd_x": load_mfma_util(name, "bwd_x")},
    }
    out["data"] = "synthetic, seeded on the GPU (torch.Generator), same scales as the workload"
    del M, R, P, dM, ws_f, ws_b, x, dx
    torch.cuda.empty_cache()
    return out


def small_configs(mpp, torch, WORKLOADS, gen_R, gen_x, reps: int = 50):
    """The two small workloads as specified: C1 (one 1024-token sequence, n=4,
    forward) and C2 (8x8 heads x 256 tokens, n=8, the step: forward from x then
    backward).  Both are launch-bound and cache-resident (128 KiB / 8 MiB), so
    they report latency, not bandwidth."""
    out = {}
    for name in ("c1", "c2"):
        w = WORKLOADS[name]
        x = torch.from_numpy(gen_x(w.B, w.H, w.T, w.n, w.sigma_off, w.sigma_diag, w.seed)).cuda()
        R = torch.from_numpy(gen_R(w.B, w.H, w.T, w.n, w.seed)).cuda()
        P = torch.empty((w.B, w.H, w.T, w.n, w.n), device="cuda")
        dM = torch.empty_like(P)
        ws_f = torch.empty(max(mpp.workspace_bytes(w.B, w.H, w.T, w.n, mpp.DIR_FWD), 256),
                           dtype=torch.uint8, device="cuda")
        ws_b = torch.empty(max(mpp.workspace_bytes(w.B, w.H, w.T, w.n, mpp.DIR_BWD), 256),
                           dtype=torch.uint8, device="cuda")
        fwd = _time(torch, lambda: mpp.scan_fwd_x(x, w.n, out=P, workspace=ws_f), reps)
        ws_ok(mpp, ws_f, w.B, w.H, w.T, w.n, mpp.DIR_FWD)
        rec = {"workload": f"{name}: B={w.B},H={w.H},T={w.T},n={w.n}",
               "plan": dict(zip(("chunk", "chunks_per_seq", "super", "ws_bytes"),
                                mpp.scan_plan(w.B, w.H, w.T, w.n, mpp.DIR_FWD))),
               "fwd_x_median_us": round(fwd, 2),
               "fwd_tokens_per_s": w.B * w.T / (fwd * 1e-6)}
        if name == "c2":
            def step():
                mpp.scan_fwd_x(x, w.n, out=P, workspace=ws_f)
                mpp.scan_bwd_x(x, P, R, out=dM, workspace=ws_b)
            st = _time(torch, step, reps)
            ws_ok(mpp, ws_b, w.B, w.H, w.T, w.n, mpp.DIR_BWD)
            rec["step_median_us"] = round(st, 2)
            rec["step_tokens_per_s"] = w.B * w.T / (st * 1e-6)
        out[name] = rec
    return out


def unfused(mpp, torch, x, R, P, dM, ws_f, ws_b, n, S, T, workload, reps: int = 10):
    """The separate kernels on the same inputs: build x -> M, scan M -> P,
    backward from M, the build's backward (x, dM -> dx), and the layer
    backward that goes from x, P, dL/dP to dL/dx in one pass (bwd_dx)."""
    M = mpp.build_inputs(x, n)
    dx = torch.empty_like(x)
    dx1 = torch.empty_like(x)
    calls = {
        "build": lambda: mpp.build_inputs(x, n, out=M),
        "fwd": lambda: mpp.scan_fwd(M, out=P, workspace=ws_f),
        "bwd": lambda: mpp.scan_bwd(M, P, R, out=dM, workspace=ws_b),
        "build_bwd": lambda: mpp.build_inputs_bwd(x, dM, out=dx),
        "bwd_dx": lambda: mpp.scan_bwd_dx(x, P, R, out=dx1, workspace=ws_b),
    }
    rec = {}
    for name, fn in calls.items():
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        avg = sum(ev[i].elapsed_time(ev[i + 1]) for i in range(reps)) / reps
        rec[name] = kernel_record(name, avg, S, T, n, workload)
    del M, dx, dx1
    return rec


def _time(torch, fn, reps):
    for _ in range(WARMUP_EXTRA):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
    return t[len(t) // 2] * 1e3  # median, microseconds


def next_rows(mpp, torch):
    """Figures for the rows beyond the core path: the scaled forward, the
    orthogonal input builds and token-by-token streaming with a carried state."""
    out = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    # scaled vs plain forward on the n = 32, 64K-token workload
    B, H, T, n = 1, 8, 65536, 32
    x = (torch.randn((B, H, T, n * n), generator=g, device="cuda") * 0.02).contiguous()
    M = mpp.build_inputs(x, n)
    ws = torch.empty(max(mpp.workspace_bytes(B, H, T, n), 256), dtype=torch.uint8, device="cuda")
    plain = _time(torch, lambda: mpp.scan_fwd(M, workspace=ws), 5)
    scaled = _time(torch, lambda: mpp.scan_fwd_ex(M, scaled=True, workspace=ws), 5)
    out["scaled_fwd"] = {"workload": "c4 shape (1x8x65536, n=32): every P_t as 2^E times a normalised matrix",
                         "median_us": round(scaled, 1), "plain_median_us": round(plain, 1),
                         "achieved_GBs": round((8 * n * n + 4) * B * H * T / (scaled * 1e-6) / 1e9, 1)}
    # orthogonal builds: fp64 arithmetic per token, Cayley 2n^3 and exp about (12 + s) * n^3 multiply-adds
    orth = {}
    for name, (B, H, T, n) in {"c2l shape, n=8": (1024, 8, 256, 8), "c4 shape, n=32": (1, 8, 65536, 32)}.items():
        x = (torch.randn((B, H, T, n * n), generator=g, device="cuda") * 0.1).contiguous()
        M = torch.empty((B, H, T, n, n), device="cuda")
        for method in ("cayley", "expm"):
            us = _time(torch, lambda: mpp.build_orthogonal(x, n, method, out=M), 5)
            fma = (2 if method == "cayley" else 12) * n ** 3 * B * H * T
            orth[f"{method}, {name}"] = {
                "median_us": round(us, 1),
                "achieved_GBs": round(8 * n * n * B * H * T / (us * 1e-6) / 1e9, 1),
                "fp64_tflops_lower_bound": round(2 * fma / (us * 1e-6) / 1e12, 2),
                "fp64_vector_peak_tflops": FP64_PEAK_TFLOPS}
        del x, M
    out["orthogonal_build"] = orth
    # streaming: one token per call for 8192 sequences of 8x8 states (a decode step)
    B, H, n = 1024, 8, 8
    xs = (torch.randn((B, H, 1, n * n), generator=g, device="cuda") * 0.1).contiguous()
    state = mpp.scan_fwd_x(xs, n)[:, :, 0].contiguous()
    us = _time(torch, lambda: mpp.scan_fwd_ex(xs, carry=state, from_x=True, n=n), 20)
    out["decode_step"] = {"workload": "8192 sequences (1024x8), n=8, one token from x with the carried state",
                          "median_us": round(us, 1), "tokens_per_s": B / (us * 1e-6)}
    torch.cuda.empty_cache()
    return out


def copy_reference(torch, gib: int = 1, reps: int = 10):
    """A plain device-to-device copy of known size on the same GPU: the practical
    streaming bandwidth this machine reaches, and the known-size kernel that scales
    the HBM traffic counters."""
    n = gib * (2 ** 30) // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        b.copy_(a)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
    med = t[len(t) // 2]
    del a, b
    torch.cuda.empty_cache()
    moved = 2 * gib * 2 ** 30
    return {"bytes_per_launch": moved, "median_us": round(med * 1e3, 1),
            "GBs": round(moved / (med * 1e-3) / 1e9, 1),
            "frac_hbm": round(moved / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel": "torch copy_ of a 1 GiB fp32 tensor"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2l")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the n=16 / n=32 forward figures")
    ap.add_argument("--extra-only", action="store_true",
                    help="only the n=16 / n=32 and next-row figures (for profiling those kernels)")
    ap.add_argument("--only", choices=("c3", "c4", "c5"),
                    help="with --extra-only: just this workload's figures (one workload per profile)")
    ap.add_argument("--summarize", choices=("trace", "traffic", "mfma", "counters"),
                    help="print the summary of the rocprofv3 CSVs under DIR... (no GPU work)")
    ap.add_argument("--profile-workload", help="with --summarize: the workload the runs covered")
    ap.add_argument("--command", action="append", default=[],
                    help="with --summarize: a command that produced DIR (repeatable)")
    ap.add_argument("dirs", nargs="*", help="with --summarize: rocprofv3 output folders")
    args = ap.parse_args()
    if args.summarize:
        if not args.profile_workload or not args.dirs:
            sys.exit("--summarize needs --profile-workload and at least one folder")
        summarize(args.summarize, args.dirs, args.profile_workload, args.command)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the MRU scan shards over independent "
              "sequences with no communication, so the benchmark measures one GPU's share; "
              f"--gpus {args.gpus} (WORLD_SIZE={world}) is not supported.", file=sys.stderr)
        sys.exit(2)

    from workloads import WORKLOADS, gen_R, gen_x

    w = WORKLOADS[args.workload]
    cpu = None
    if not args.no_cpu_baseline and not args.extra_only:
        cpu, cpu_ref = cpu_leg(w, args.cpu_seconds)  # before anything touches the GPU

    import numpy as np
    import torch

    import matrix_prefix_product_amd as mpp

    B, H, T, n = w.B, w.H, w.T, w.n
    S = B * H
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.extra_only:
        c3, c4, c5 = WORKLOADS["c3"], WORKLOADS["c4"], WORKLOADS["c5"]
        runs = {
            "n16": lambda: fwd_only(mpp, torch, "c3", c3.B, c3.H, c3.T, c3.n, c3.sigma_off, c3.sigma_diag, 20, 3),
            "n32": lambda: fwd_only(mpp, torch, "c4", c4.B, c4.H, c4.T, c4.n, c4.sigma_off, c4.sigma_diag, 5, 4),
            "n16_fwd_bwd": lambda: fwd_bwd(mpp, torch, "c5", c5.B, c5.H, c5.T, c5.n, c5.sigma_off,
                                           c5.sigma_diag, 10, 5),
            "small": lambda: small_configs(mpp, torch, WORKLOADS, gen_R, gen_x),
            "next": lambda: next_rows(mpp, torch),
        }
        if args.only:
            runs = {k: v for k, v in runs.items() if k == {"c3": "n16", "c4": "n32", "c5": "n16_fwd_bwd"}[args.only]}
        extra = {}
        for k, fn in runs.items():
            extra[k] = fn()
            print(f"# {k} done", file=sys.stderr, flush=True)
        print(json.dumps(extra), flush=True)
        return

    x = torch.from_numpy(gen_x(B, H, T, n, w.sigma_off, w.sigma_diag, w.seed)).to(dev)
    R = torch.from_numpy(gen_R(B, H, T, n, w.seed)).to(dev)
    if n not in mpp.FUSED_N:
        sys.exit(f"the step starts from raw token vectors, available for n in {mpp.FUSED_N}")
    P = torch.empty((B, H, T, n, n), device=dev)
    dM = torch.empty_like(P)
    ws_f = torch.empty(max(mpp.workspace_bytes(B, H, T, n, mpp.DIR_FWD), 256), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(mpp.workspace_bytes(B, H, T, n, mpp.DIR_BWD), 256), dtype=torch.uint8, device=dev)

    # events are recorded on torch's current stream, the stream every call below launches on
    def step(ev=None):
        if ev is not None:
            ev[0].record()
        mpp.scan_fwd_x(x, n, out=P, workspace=ws_f)
        if ev is not None:
            ev[1].record()
        mpp.scan_bwd_x(x, P, R, out=dM, workspace=ws_b)
        if ev is not None:
            ev[2].record()

    # The separate kernels run first: besides their own figures they bring the
    # GPU past the clock transient that follows a start from idle (launched back
    # to back from idle, this step takes 540 us, then up to 623 us by the ninth
    # step, and settles at ~536 us from the thirtieth on), so that the --warmup
    # steps and the timed steps see the sustained rate.
    unfused_rec = unfused(mpp, torch, x, R, P, dM, ws_f, ws_b, n, S, T, w.name)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    if cpu is not None:
        rows = cpu_ref[0].shape[0]
        gpu_rows = (P[:rows].cpu().numpy(), dM[:rows].cpu().numpy())
    ms_per_step = total_ms / args.steps
    per = {k: [] for k in ("fwd_x", "bwd_x")}
    for e in evs:
        per["fwd_x"].append(e[0].elapsed_time(e[1]))
        per["bwd_x"].append(e[1].elapsed_time(e[2]))
    kernels = {k: kernel_record(k, float(np.mean(v)), S, T, n, w.name) for k, v in per.items()}
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
    dk = kernels[dom]
    tokens_per_s = B * T / (ms_per_step * 1e-3)

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64" if n == 16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: char-LM-shaped MRU layer, B={B}, H={H} heads, T={T}, n={n} "
                        "(d_model 512 as 8 heads of 8x8); one step = forward scan from the raw "
                        "token vectors (LDU build fused) + backward scan to dL/dM",
            "B": B, "H": H, "T": T, "n": n,
            "fwd_plan": dict(zip(("chunk", "chunks_per_seq", "super", "ws_bytes"),
                                 mpp.scan_plan(B, H, T, n, mpp.DIR_FWD))),
            "bwd_plan": dict(zip(("chunk", "chunks_per_seq", "super", "ws_bytes"),
                                 mpp.scan_plan(B, H, T, n, mpp.DIR_BWD))),
        },
        "roofline": {
            "kernel": dom,
            "bound": "hbm",
            "achieved": dk["achieved_GBs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": dk["frac_hbm"],
            "traffic": dk["traffic"],
            "algorithmic_bytes_per_launch": dk["algorithmic_bytes"],
            "frac_traffic": dk["frac_hbm_traffic"],
            "design_bytes_per_launch": dk["design_bytes"],
            "basis": "achieved = algorithmic bytes per launch (16 n^2 per token-head for the "
                     "backward: x, P, dL/dP read and dL/dM written) / the kernel's mean launch "
                     "time; frac_traffic uses the counted HBM bytes instead",
        },
        "kernels": kernels,
        "wall_s_timed": round(wall, 4),
        "preconditioning": "before the warmup steps the unfused comparison kernels of the same "
                           "workload run (5 kernels x 11 launches, ~20 ms of GPU work)",
    }
    # every look-back wait of the timed scans completed (multi-chunk plans only)
    ws_ok(mpp, ws_f, B, H, T, n, mpp.DIR_FWD)
    ws_ok(mpp, ws_b, B, H, T, n, mpp.DIR_BWD)
    out["unfused"] = unfused_rec
    del x, R, P, dM, ws_f, ws_b
    torch.cuda.empty_cache()
    out["copy_reference"] = copy_reference(torch)

    if not args.no_extra:
        c3, c4, c5 = WORKLOADS["c3"], WORKLOADS["c4"], WORKLOADS["c5"]
        out["n16"] = fwd_only(mpp, torch, "c3", c3.B, c3.H, c3.T, c3.n, c3.sigma_off, c3.sigma_diag, 20, 3)
        out["n32"] = fwd_only(mpp, torch, "c4", c4.B, c4.H, c4.T, c4.n, c4.sigma_off, c4.sigma_diag, 5, 4)
        out["n16_fwd_bwd"] = fwd_bwd(mpp, torch, "c5", c5.B, c5.H, c5.T, c5.n, c5.sigma_off,
                                     c5.sigma_diag, 10, 5)
        out["small"] = small_configs(mpp, torch, WORKLOADS, gen_R, gen_x)
        out["next"] = next_rows(mpp, torch)
    if cpu is not None:
        cpu["parity_sample"] = cpu_parity(cpu_ref, gpu_rows)
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
