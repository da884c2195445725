#!/usr/bin/env python3
"""Throughput of the quaternion cumulative-product scan, forward + backward, on
one MI355X.

A step is one pass of the whole path over one batch of synthetic input that is
already resident in HBM: the forward (q, init -> cum, writing the saved
boundary state) then the backward (q, init, d_cum, boundary state -> d_q,
d_init).  Default workload: b=8, s=4096, h=32, j=32, float32 storage
(33,554,432 quaternions, 512 MiB per [b,s,h,j,4] tensor), seeded unit
quaternions.

Timing: W untimed warm-up steps, continued until --settle-ms of sustained
load has passed (the first tens of ms after idle run at unsettled clocks),
then K timed steps between two device synchronisations.  Inside the timed
region HIP events bracket every N-th backward launch on its stream (the
roofline figure; N = --event-every, 4 by default, since each event pair idles
the GPU for a few us); a short loop after it brackets both kernels for the
forward / backward split.

Reported value: algorithmic bytes per step (32 B/quaternion forward + 48 B
backward, plus 16 B per column for init and d_init) / wall time per step.
The line also reports, timed after the main region, the final-carry mode
(the forward saves only cum[:, s-1] per column and the backward rebuilds the
rest from the end of the sequence) and the leaves-only mode (nothing saved;
the backward re-derives the boundary state from q).
The last stdout line is one JSON record; diagnostics go to stderr.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "quat cumprod fwd+bwd GB/s and % HBM peak, b8·s4096·h32·j32 fp32"
HBM_PEAK_GBPS = 8000.0
# Sources that define the kernels and their launch shapes (code, tile geometry, planning).
KERNEL_SOURCES = [os.path.join(ROOT, "quaternion_cumprod_autodiff_amd", "csrc", f)
                  for f in ("qc_kernels.hip", "qc_internal.hpp", "qc_abi.cpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_headline.txt")
WORKLOAD_KEY = "headline b8 s4096 h32 j32 f32 I/O, forward + backward"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_kv(path: str) -> dict:
    out = {}
    with open(path) as f:
        for ln in f:
            if "=" in ln and not ln.lstrip().startswith("#"):
                k, v = ln.split("=", 1)
                out[k.strip()] = v.strip()
    return out


def load_traffic(workload_key: str):
    """HBM bytes per backward launch from the committed rocprofv3 counter
    summary, or None when missing or taken on a different kernel source."""
    try:
        rec = read_kv(TRAFFIC_FILE)
    except OSError:
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha() or rec.get("workload") != workload_key:
        return None
    return float(rec["bwd_hbm_bytes_per_launch"])


def summarize_traffic(pmc_dir: str, copy_bytes: float):
    """Scale rocprofv3 FETCH_SIZE / WRITE_SIZE readings (KiB per dispatch) by
    what the same counters read for a plain device copy of known size, and
    write the per-launch HBM bytes of the scan kernels to profiles/."""
    import csv
    import statistics

    def per_kernel(run, counter):
        vals = {}
        path = os.path.join(pmc_dir, run, "run_counter_collection.csv")
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            # The forward that writes cum (not the boundary-state pass of a
            # backward without saved state, the ", false>" instantiation).
            key = ("bwd" if "bwd_chunked_kernel" in name
                   else "fwd" if "fwd_chunked_kernel" in name and ", false>" not in name
                   else "copy" if "copyBuffer" in name else None)
            if key:
                vals.setdefault(key, []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: statistics.median(v) for k, v in vals.items()}

    f, w = per_kernel("FETCH_SIZE", "FETCH_SIZE"), per_kernel("WRITE_SIZE", "WRITE_SIZE")
    fs = copy_bytes / per_kernel("copy_FETCH_SIZE", "FETCH_SIZE")["copy"]
    ws = copy_bytes / per_kernel("copy_WRITE_SIZE", "WRITE_SIZE")["copy"]
    rec = {
        "workload": WORKLOAD_KEY,
        "kernel_source_sha256": kernel_source_sha(),
        "fetch_scale": f"{fs:.4f}", "write_scale": f"{ws:.4f}",
        "fwd_fetch_bytes": f"{f['fwd'] * fs:.0f}", "fwd_write_bytes": f"{w['fwd'] * ws:.0f}",
        "bwd_fetch_bytes": f"{f['bwd'] * fs:.0f}", "bwd_write_bytes": f"{w['bwd'] * ws:.0f}",
        "fwd_hbm_bytes_per_launch": f"{f['fwd'] * fs + w['fwd'] * ws:.0f}",
        "bwd_hbm_bytes_per_launch": f"{f['bwd'] * fs + w['bwd'] * ws:.0f}",
    }
    with open(TRAFFIC_FILE, "w") as out:
        out.write("# HBM traffic per launch of the scan kernels, headline workload (b8 s4096 h32 j32, f32 I/O).\n")
        out.write("# Counters: rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (KiB per dispatch), each\n")
        out.write("# scaled by bytes / reading of the same counter for a plain device copy of one tensor.\n")
        out.write("# Commands (run from /tmp, TMPDIR=/tmp, R = repository root, OUT = an output directory):\n")
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            out.write(f"#   rocprofv3 --pmc {ctr} --output-format csv -d $OUT/pmc/{ctr} -o run -- "
                      f"python3 $R/bench.py --steps 2 --warmup 1 --settle-ms 0 --leaves-steps 0 --no-cpu-baseline\n")
            out.write(f"#   rocprofv3 --pmc {ctr} --output-format csv -d $OUT/pmc/copy_{ctr} -o run -- "
                      f"python3 $R/bench.py --copy-calibration --steps 2 --warmup 1\n")
        out.write(f"#   python3 $R/bench.py --summarize-traffic $OUT/pmc\n")
        for k, v in rec.items():
            out.write(f"{k} = {v}\n")
    print(json.dumps(rec))


def cpu_baseline(inp, min_seconds: float = 10.0):
    """The float64 oracle timed on the host cores on a bounded sample: the
    first batch entry of the workload (all h*j columns, all s steps)."""
    import numpy as np

    import oracle
    q = inp.q[:1].astype(np.float64)
    init = inp.init[:1].astype(np.float64)
    d = inp.d_cum[:1].astype(np.float64)
    n = q.shape[0] * q.shape[1] * q.shape[2] * q.shape[3]
    cols = q.shape[2] * q.shape[3]
    threads = oracle.threads(0)
    oracle.fwd(q[:, :64], init)             # load and warm up
    reps, t_total, each = 0, 0.0, []
    while t_total < min_seconds or reps == 0:
        t0 = time.perf_counter()
        oracle.fwd(q, init, threads)
        t1 = time.perf_counter()
        oracle.bwd(q, init, d, threads)
        t_total += time.perf_counter() - t0
        each.append((t1 - t0, time.perf_counter() - t1))
        reps += 1
    per_pass = t_total / reps
    gbps = (80.0 * n + 32.0 * cols) / per_pass / 1e9
    fwd_med = float(np.median([f for f, _ in each]))    # forward and backward separately, medians
    bwd_med = float(np.median([b for _, b in each]))
    # One thread on 1/16 of the same sample (the first 64 columns), same byte formula.
    s_len = q.shape[1]
    q1 = np.ascontiguousarray(q.reshape(1, s_len, cols, 4)[:, :, :64])
    i1 = np.ascontiguousarray(init.reshape(1, cols, 4)[:, :64])
    d1 = np.ascontiguousarray(d.reshape(1, s_len, cols, 4)[:, :, :64])
    n1, reps1, t1 = q1.shape[1] * q1.shape[2], 0, 0.0
    while t1 < min_seconds / 4 or reps1 == 0:
        t0 = time.perf_counter()
        oracle.fwd(q1, i1, 1)
        oracle.bwd(q1, i1, d1, 1)
        t1 += time.perf_counter() - t0
        reps1 += 1
    gbps1 = (80.0 * n1 + 32.0 * q1.shape[2]) / (t1 / reps1) / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"batch entry 0 of the workload ({cols} columns x {q.shape[1]} steps = {n} quaternions), "
                      f"float64 forward + reverse-recurrence backward, {reps} pass(es), {per_pass:.2f} s per pass",
            "cpu_model": cpu_model(),
            "fwd_GBps": round((32.0 * n + 16.0 * cols) / fwd_med / 1e9, 4),
            "bwd_GBps": round((48.0 * n + 32.0 * cols) / bwd_med / 1e9, 4),
            "fwd_s_median": round(fwd_med, 5), "bwd_s_median": round(bwd_med, 5),
            "one_thread": {"value": round(gbps1, 4), "unit": "GB/s", "cores": 1,
                           "sample": f"the first 64 columns of the same sample ({n1} quaternions), "
                                     f"{reps1} pass(es), {t1 / reps1:.3f} s per pass"}}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_calibration(nbytes: int, steps: int, warmup: int):
    """Plain device-to-device copy of a tensor of known size (HBM ceiling and
    the reference point for scaling hardware byte counters)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    return 2.0 * nbytes / dt / 1e9, dt


def copy_ceiling(nbytes: int, steps: int = 20):
    """The hand-written streaming copy (include/qc_bench.h) of one nbytes
    tensor: best rate over a few grid sizes (blocks per compute unit), each
    timed over `steps` copies between device synchronisations."""
    import torch

    from quaternion_cumprod_autodiff_amd import capi
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    best = None
    for bpc in (2, 4, 8, 16):
        for _ in range(5):
            capi.stream_copy(src, dst, blocks_per_cu=bpc)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            capi.stream_copy(src, dst, blocks_per_cu=bpc)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        gbps = 2.0 * nbytes / dt / 1e9
        if best is None or gbps > best[0]:
            best = (gbps, dt, bpc)
    if not torch.equal(src, dst):
        raise RuntimeError("the streaming copy produced a different tensor")
    torch_gbps, torch_dt = copy_calibration(nbytes, steps, 5)
    return {"value": round(best[0], 1), "unit": "GB/s", "ms": round(best[1] * 1e3, 4),
            "kind": f"qc_stream_copy of one {nbytes} B tensor (read + write), {best[2]} blocks per CU, "
                    f"best of 2/4/8/16, {steps} timed",
            "torch_copy": {"value": round(torch_gbps, 1), "ms": round(torch_dt * 1e3, 4)}}


# ------------------------------------------------------------- generic scan
# The scan VJP of include/qc_scan.h (add or quaternion body, one column per
# thread).  Workload: the page's scan test length, 129 steps, over enough
# columns that every lane of the chip has one (2^20 quaternion columns,
# 2^22 scalar ones: 2.16 GB per [b, s, m, w] tensor either way).
SCAN_WORKLOADS = {"quat": (1, 129, 1 << 20), "add": (1, 129, 1 << 22)}


def scan_schedule_bytes(body: str, sched, lo: int, hi: int, ebytes: int, cols: int, w: int) -> int:
    """Algorithmic bytes of schedule records [lo, hi): every body evaluation
    reads one x; a reversed step also reads its upstream cotangent and writes
    its d_x, and reads x only where the body's VJP depends on it (the
    quaternion body; the add body's Jacobians are constant); a snapshot store
    or load moves one float64 carry."""
    acts = sched.actions[lo:hi].numpy()
    op = acts[:, 0]
    adv = int((acts[op == 3, 2] - acts[op == 3, 1]).sum())
    rev = int((op == 4).sum())
    snap = int(((op == 1) | (op == 2)).sum())
    rev_bytes = 3 if body == "quat" else 2
    return cols * (ebytes * (adv + rev_bytes * rev) + 8 * w * snap)


SCAN_SOURCES = [os.path.join(ROOT, "quaternion_cumprod_autodiff_amd", "csrc", "qc_scan.hip")]
SCAN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_scan_quat.txt")


def scan_source_sha() -> str:
    h = hashlib.sha256()
    for path in SCAN_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def summarize_scan_traffic(pmc_dir: str, fetch_scale: float, write_scale: float):
    """HBM bytes per launch of the quaternion-body scan kernels (trajectory
    mode) from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of ``--scan quat``,
    scaled like the headline's (the copy calibration's factors)."""
    import csv
    import statistics

    def per_kernel(counter):
        vals = {}
        path = os.path.join(pmc_dir, counter, "run_counter_collection.csv")
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = ("bwd" if "scan_bwd_trajectory_kernel" in name
                   else "fwd" if "scan_fwd_kernel" in name else None)
            if key:
                vals.setdefault(key, []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: statistics.median(v) for k, v in vals.items()}

    f, w = per_kernel("FETCH_SIZE"), per_kernel("WRITE_SIZE")
    b, s, m = SCAN_WORKLOADS["quat"]
    rec = {
        "workload": f"scan quat b{b} s{s} m{m} f32 I/O, forward + VJP (trajectory)",
        "kernel_source_sha256": scan_source_sha(),
        "fetch_scale": f"{fetch_scale:.4f}", "write_scale": f"{write_scale:.4f}",
        "fwd_fetch_bytes": f"{f['fwd'] * fetch_scale:.0f}", "fwd_write_bytes": f"{w['fwd'] * write_scale:.0f}",
        "bwd_fetch_bytes": f"{f['bwd'] * fetch_scale:.0f}", "bwd_write_bytes": f"{w['bwd'] * write_scale:.0f}",
        "fwd_hbm_bytes_per_launch": f"{f['fwd'] * fetch_scale + w['fwd'] * write_scale:.0f}",
        "bwd_hbm_bytes_per_launch": f"{f['bwd'] * fetch_scale + w['bwd'] * write_scale:.0f}",
    }
    with open(SCAN_TRAFFIC_FILE, "w") as out:
        out.write("# HBM traffic per launch of the generic scan kernels, quaternion body, trajectory mode.\n")
        out.write("# Counters: rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (KiB per dispatch), scaled by\n")
        out.write("# the factors of the plain-copy calibration in traffic_headline.txt.\n")
        out.write("# Commands (run from /tmp, TMPDIR=/tmp, R = repository root, OUT = an output directory):\n")
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            out.write(f"#   rocprofv3 --pmc {ctr} --output-format csv -d $OUT/pmc_scan/{ctr} -o run -- "
                      f"python3 $R/bench.py --scan quat --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline\n")
        out.write("#   python3 $R/bench.py --summarize-scan-traffic $OUT/pmc_scan\n")
        for k, v in rec.items():
            out.write(f"{k} = {v}\n")
    print(json.dumps(rec))


def load_scan_traffic(workload_key: str):
    try:
        rec = read_kv(SCAN_TRAFFIC_FILE)
    except OSError:
        return None
    if rec.get("kernel_source_sha256") != scan_source_sha() or rec.get("workload") != workload_key:
        return None
    return float(rec["bwd_hbm_bytes_per_launch"])


def scan_cpu_baseline(body: str, xs, init, up, min_seconds: float = 10.0):
    """The float64 numpy oracle of the generic scan on the first 4096 columns."""
    import oracle
    cols = min(4096, xs.shape[2])
    x = xs[:, :, :cols].double().cpu().numpy()
    i0 = init[:, :cols].double().cpu().numpy()
    u = up[:, :, :cols].double().cpu().numpy()
    w = x.shape[-1]
    n = x.shape[0] * x.shape[1] * cols
    reps, t_total = 0, 0.0
    while t_total < min_seconds or reps == 0:
        t0 = time.perf_counter()
        oracle.scan_fwd(body, x, i0)
        oracle.scan_bwd(body, x, i0, u)
        t_total += time.perf_counter() - t0
        reps += 1
    per_pass = t_total / reps
    per_elem, per_col = (6, 3) if body == "quat" else (4, 2)   # the device leg's trajectory-mode bytes
    gbps = 4 * w * (per_elem * n + per_col * x.shape[0] * cols) / per_pass / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the first {cols} columns x {x.shape[1]} steps ({n} elements), float64 numpy forward + "
                      f"reverse sweep over the saved trajectory, {reps} pass(es), {per_pass:.3f} s per pass",
            "cpu_model": cpu_model()}


def scan_bench(args):
    """One step = the scan's forward (ys, plus the snapshots with --scan-k) and
    its VJP, from the saved trajectory (--scan-k 0) or from k snapshots."""
    import numpy as np
    import torch

    from quaternion_cumprod_autodiff_amd import capi
    from quaternion_cumprod_autodiff_amd.inputs import SCAN_WIDTH, make_generic_scan_inputs_device

    body, k = args.scan, args.scan_k
    b, s, m = SCAN_WORKLOADS[body]
    w = SCAN_WIDTH[body]
    eb, cols = 4 * w, b * m
    n = cols * s
    dev = torch.device("cuda:0")
    xs, init, up = make_generic_scan_inputs_device(body, b, s, m, 0, dev)
    ys = torch.empty_like(xs)
    d_xs, d_init = torch.empty_like(xs), torch.empty_like(init)
    if k > 0:
        sch = capi.ScanSchedule(s, k)
        snaps = capi.new_snapshots(body, xs, k)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        fwd_bytes = 2 * eb * n + eb * cols + scan_schedule_bytes(body, sch, 0, sch.bwd_start, eb, cols, w)
        bwd_bytes = (scan_schedule_bytes(body, sch, sch.bwd_start, sch.n_actions, eb, cols, w)
                     + 8 * w * cols + eb * cols)      # resume load, d_init
        kernel = "scan_bwd_checkpointed_kernel"

        def fwd():
            capi.scan_fwd(body, xs, init, ys, schedule=sch, snaps=snaps)

        def bwd():
            capi.scan_bwd_checkpointed(body, xs, init, up, sch, snaps, after_forward=True, status=status,
                                       d_xs=d_xs, d_init=d_init)
    else:
        sch = status = None
        fwd_bytes = 2 * eb * n + eb * cols
        # quat: xs, ys[t-1] (init at t = 0), upstream, d_xs, d_init.  add: the
        # VJP depends on neither x nor the carries, so upstream, d_xs, d_init.
        bwd_bytes = eb * (4 * n + cols) if body == "quat" else eb * (2 * n + cols)
        kernel = "scan_bwd_trajectory_kernel"

        def fwd():
            capi.scan_fwd(body, xs, init, ys)

        def bwd():
            capi.scan_bwd_trajectory(body, xs, init, ys, up, d_xs=d_xs, d_init=d_init)

    warm, t0 = 0, time.perf_counter()
    while warm < args.warmup or (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        fwd()
        bwd()
        warm += 1
        if warm % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731
    every = max(1, args.event_every)
    be = {i: (ev(), ev()) for i in range(every - 1, args.steps, every)}
    t0 = time.perf_counter()
    for i in range(args.steps):
        fwd()
        if i in be:
            be[i][0].record()
            bwd()
            be[i][1].record()
        else:
            bwd()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if status is not None and int(status.item()) != 0:
        raise RuntimeError("the device refused a schedule record")
    bwd_ms = float(np.mean([a.elapsed_time(c) for a, c in be.values()]))
    diag = [(ev(), ev()) for _ in range(10)]
    for f0, f1 in diag:
        f0.record()
        fwd()
        f1.record()
    torch.cuda.synchronize()
    fwd_ms = float(np.median([a.elapsed_time(c) for a, c in diag]))
    ms_step = wall / args.steps * 1e3
    value = (fwd_bytes + bwd_bytes) / (ms_step * 1e-3) / 1e9
    bwd_gbps = bwd_bytes / (bwd_ms * 1e-3) / 1e9
    mode = f"checkpointed k={k}" if k > 0 else "trajectory"
    workload = f"scan {body} b{b} s{s} m{m} f32 I/O, forward + VJP ({mode})"
    rec = {
        "metric": f"generic scan fwd+bwd GB/s, {body} body, b{b} s{s} m{m} f32 ({mode})",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64", "data": "synthetic",
        "config": {"workload": workload,
                   "b": b, "s": s, "m": m, "body": body, "mode": mode},
        "hbm_frac": round(value / HBM_PEAK_GBPS, 4), "elements_per_s": round(n / (ms_step * 1e-3), 1),
        "fwd_bytes": fwd_bytes, "bwd_bytes": bwd_bytes,
        "bwd_ms": round(bwd_ms, 4), "bwd_launches_timed": len(be), "diag_fwd_ms": round(fwd_ms, 4),
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(bwd_gbps, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(bwd_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": load_scan_traffic(workload)},
        "cpu_baseline": None,
    }
    if sch is not None:
        rec["schedule"] = {"k": k, "records": sch.n_actions, "body_evaluations": sch.forward_steps,
                           "in_forward": sch.prefix_steps}
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        rec["cpu_baseline"] = scan_cpu_baseline(body, xs, init, up)
    print(json.dumps(rec), flush=True)


# -------------------------------------------------------- Gated DeltaNet-2
# The recurrence of include/gdn2.h at the page's training head shape (latent
# 64, dense 128) over 8 x 16 heads and 2048 steps, in chunk-WY form on fp32
# MFMA at chunks of 32 steps (chunks of 16 or 32 select that form; any other
# chunk runs the step-by-step recurrent kernels).
GDN2_WORKLOAD = (8, 16, 2048, 64, 128, 32)
FP32_MFMA_PEAK_TFLOPS = 157.3
GDN2_SOURCES = [os.path.join(ROOT, "quaternion_cumprod_autodiff_amd", "csrc", f)
                for f in ("gdn2.hip", "gdn2_wy.hip", "gdn2_internal.hpp")]
GDN2_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gdn2.txt")


def gdn2_source_sha() -> str:
    h = hashlib.sha256()
    for path in GDN2_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def gdn2_bytes_and_flops(B, H, T, L, D, C):
    """Algorithmic bytes and flops of one forward and one VJP (float32).

    Bytes: every input read once, every output written once (the saved
    boundary states, factor records and updates, and the backward's scratch,
    are the method's own state and are not counted).

    Flops: the chunk-WY form at chunk C, counted per chunk of every head as
    multiply-adds (2 flops each), a triangular product as half its dense size:
      forward  A = M Wb^T and Bq = Qc Wb^T: C^2 L;  T = (I + A)^-1: C^3 / 6;
               M S0, Qc S0, Kt^T U: 3 C L D;  T rhs and Bq U: C^2 D
      VJP      Bq^T dO, T^T dU, dO U^T, drhs U^T: 2 C^2 D;
               Kt dS, Qc^T dO, M^T drhs, dO S0^T, drhs S0^T, U dSc^T: 6 C L D;
               dBq Wb, dA Wb, dBq^T Qc, dA^T M: 2 C^2 L
    with ceil(T / C) chunks per head."""
    heads = B * H
    chunks = heads * ((T + C - 1) // C)
    fwd_bytes = 4 * heads * (T * (4 * L + 2 * D) + L * D + T * D + L * D)
    bwd_bytes = 4 * heads * (T * (4 * L + 3 * D) + T * (4 * L + 2 * D) + L * D)
    fwd_mac = C * C * L + C ** 3 / 6 + 3 * C * L * D + C * C * D
    bwd_mac = 2 * C * C * D + 6 * C * L * D + 2 * C * C * L
    return fwd_bytes, bwd_bytes, int(2 * fwd_mac * chunks), int(2 * bwd_mac * chunks)


def load_gdn2_traffic(workload_key: str):
    """HBM bytes per VJP (both backward launches) from the committed counter
    summary, or None when missing or taken on different kernel sources."""
    try:
        rec = read_kv(GDN2_TRAFFIC_FILE)
    except OSError:
        return None
    if rec.get("kernel_source_sha256") != gdn2_source_sha() or rec.get("workload") != workload_key:
        return None
    return float(rec["bwd_hbm_bytes"])


def summarize_gdn2_traffic(pmc_dir: str, workload_key: str):
    """profiles/traffic_gdn2.txt from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of
    --gdn2, scaled by the plain-copy calibration of traffic_headline.txt."""
    import csv
    import statistics
    cal = read_kv(TRAFFIC_FILE)
    fs, ws = float(cal["fetch_scale"]), float(cal["write_scale"])

    def per_kernel(counter):
        vals = {}
        for r in csv.DictReader(open(os.path.join(pmc_dir, counter, "run_counter_collection.csv"))):
            if r["Counter_Name"] != counter or "wy_" not in r["Kernel_Name"]:
                continue
            name = r["Kernel_Name"].split("(anonymous namespace)::")[-1].split("(")[0]
            vals.setdefault(name, []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: statistics.median(v) for k, v in vals.items()}

    f, w = per_kernel("FETCH_SIZE"), per_kernel("WRITE_SIZE")
    B, H, T, L, D, C = GDN2_WORKLOAD
    fb, bb, _, _ = gdn2_bytes_and_flops(B, H, T, L, D, C)
    fwd = sum(f[k] * fs + w.get(k, 0.0) * ws for k in f if "fwd" in k or "factor" in k)
    bwd = sum(f[k] * fs + w.get(k, 0.0) * ws for k in f if "bwd" in k)
    with open(GDN2_TRAFFIC_FILE, "w") as out:
        out.write("# HBM traffic of the Gated DeltaNet-2 chunk-WY kernels, bench workload.\n")
        out.write("# Counters: rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (KiB per dispatch), scaled by\n")
        out.write("# the factors of the plain-copy calibration in traffic_headline.txt; median over the run.\n")
        out.write("# Commands (run from /tmp, TMPDIR=/tmp, R = repository root, OUT = an output directory):\n")
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            out.write(f"#   rocprofv3 --pmc {ctr} --output-format csv -d $OUT/pmc_gdn2/{ctr} -o run -- "
                      f"python3 $R/bench.py --gdn2 --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline\n")
        out.write("#   python3 $R/bench.py --summarize-gdn2-traffic $OUT/pmc_gdn2\n")
        out.write(f"workload = {workload_key}\n")
        out.write(f"kernel_source_sha256 = {gdn2_source_sha()}\n")
        for k in sorted(f):
            out.write(f"{k}_fetch_bytes = {f[k] * fs:.0f}\n{k}_write_bytes = {w.get(k, 0.0) * ws:.0f}\n")
        out.write(f"fwd_hbm_bytes = {fwd:.0f}\nfwd_algorithmic_bytes = {fb}\nfwd_ratio = {fwd / fb:.3f}\n")
        out.write(f"bwd_hbm_bytes = {bwd:.0f}\nbwd_algorithmic_bytes = {bb}\nbwd_ratio = {bwd / bb:.3f}\n")
    print(open(GDN2_TRAFFIC_FILE).read())


def gdn2_bench(args):
    import numpy as np
    import torch

    from quaternion_cumprod_autodiff_amd import capi

    B, H, T, L, D, chunk = GDN2_WORKLOAD
    if args.gdn2_chunk:
        chunk = args.gdn2_chunk
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(0)
    ins = [torch.randn((B, H, T, L), device=dev, generator=g),
           torch.randn((B, H, T, L), device=dev, generator=g) / L ** 0.5,
           torch.randn((B, H, T, D), device=dev, generator=g),
           torch.rand((B, H, T, L), device=dev, generator=g),
           torch.rand((B, H, T, D), device=dev, generator=g),
           torch.rand((B, H, T, L), device=dev, generator=g) - 1.2,
           torch.randn((B, H, L, D), device=dev, generator=g)]
    d_ctx = torch.randn((B, H, T, D), device=dev, generator=g)
    out = {}

    def fwd():
        out["f"] = capi.gdn2_fwd(*ins, chunk=chunk)

    def bwd():
        capi.gdn2_bwd(*ins[:6], out["f"][2], d_ctx, chunk=chunk)

    warm, t0 = 0, time.perf_counter()
    while warm < args.warmup or (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        fwd()
        bwd()
        warm += 1
        torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731
    steps = max(1, args.steps)
    evs = [(ev(), ev(), ev()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in evs:
        e0.record()
        fwd()
        e1.record()
        bwd()
        e2.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    fwd_ms = float(np.median([a.elapsed_time(b) for a, b, _ in evs]))
    bwd_ms = float(np.median([b.elapsed_time(c) for _, b, c in evs]))
    fb, bb, ff, bf = gdn2_bytes_and_flops(B, H, T, L, D, chunk)
    wy = chunk in (16, 32)
    tflops = bf / (bwd_ms * 1e-3) / 1e12
    workload = f"gdn2 b{B} h{H} t{T} latent{L} dense{D} chunk{chunk} f32, forward + VJP"
    traffic = load_gdn2_traffic(workload) if wy else None
    traffic_gbps = traffic / (bwd_ms * 1e-3) / 1e9 if traffic else None
    rec = {
        "metric": f"Gated DeltaNet-2 fwd+bwd GB/s, b{B} h{H} t{T} latent{L} dense{D} fp32",
        "value": round((fb + bb) / wall / 1e9, 3), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": workload, "B": B, "H": H, "T": T, "L": L, "D": D, "chunk": chunk,
                   "form": "chunk-WY, fp32 MFMA" if wy else "step-by-step recurrence"},
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "fwd_bytes": fb, "bwd_bytes": bb, "fwd_flops": ff, "bwd_flops": bf,
        "fwd_tflops": round(ff / (fwd_ms * 1e-3) / 1e12, 3),
        "head_steps_per_s": round(B * H * T / wall, 1),
        "roofline": {"bound": "mfma" if wy else "alu",
                     "kernel": "gdn2_bwd (wy_bwd_carry_strip_kernel + wy_bwd_grad_kernel)" if wy else "gdn2_bwd_kernel",
                     "achieved": round(tflops, 3), "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / FP32_MFMA_PEAK_TFLOPS, 5),
                     "flops_per_launch": bf,
                     "traffic": traffic,
                     # The same VJP seen from HBM: its measured bytes over its time.
                     "traffic_GBps": round(traffic_gbps, 1) if traffic else None,
                     "traffic_frac_of_hbm_peak": round(traffic_gbps / HBM_PEAK_GBPS, 4) if traffic else None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        rec["cpu_baseline"] = gdn2_cpu_baseline([x.cpu().numpy() for x in ins], d_ctx.cpu().numpy(), (fb + bb))
    print(json.dumps(rec), flush=True)


def gdn2_cpu_baseline(arrays, d_ctx, total_bytes, min_seconds: float = 10.0):
    """The float64 numpy oracle (forward + VJP) on the first head's first
    256 steps, scaled to the same byte count per head-step."""
    import oracle
    B, H, T, L = arrays[0].shape
    ts = min(T, 256)
    sample = [a[:1, :1, :ts] if a.ndim == 4 and a.shape[2] == T else a[:1, :1] for a in arrays]
    dc = d_ctx[:1, :1, :ts]
    reps, t_total = 0, 0.0
    while t_total < min_seconds or reps == 0:
        t0 = time.perf_counter()
        oracle.gdn2_fwd(*sample)
        oracle.gdn2_bwd(*sample, dc)
        t_total += time.perf_counter() - t0
        reps += 1
    per_pass = t_total / reps
    bytes_per_head_step = total_bytes / (B * H * T)
    return {"value": round(bytes_per_head_step * ts / per_pass / 1e9, 6), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"one head, the first {ts} steps, float64 numpy forward + VJP over the saved states, "
                      f"{reps} pass(es), {per_pass:.3f} s per pass"}


# ---------------------------------------------------------------- per config
def all_configs_bench(args):
    """One JSON line per named workload and backward mode: forward, backward
    and whole-step rates (algorithmic bytes / time), elements per second and
    fractions of 8 TB/s.  Step time is wall time over --steps steps between
    device synchronisations; the forward and backward times are medians of
    20 event-bracketed launches each, after the timed steps."""
    import numpy as np
    import torch

    from quaternion_cumprod_autodiff_amd import capi
    from quaternion_cumprod_autodiff_amd.inputs import CONFIGS, make_inputs

    dev = torch.device("cuda:0")
    names = args.configs.split(",") if args.configs else list(CONFIGS)
    shards = max(1, args.seq_shards)
    for name in names:
        b, s, h, j, recipe, io = CONFIGS[name]
        # One GPU's share of a sequence-sharded run: the first s / shards steps.
        s = -(-s // shards)
        n, cols = b * s * h * j, b * h * j
        io_bytes = 16 if io == "f32" else 8
        inp = make_inputs(b, s, h, j, recipe, io, seed=0, want_f64=False)

        def up(a):
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16 if io == "bf16" else np.float32)).to(dev)
            return t.view(torch.bfloat16) if io == "bf16" else t

        q, init, d_cum = up(inp.q), up(inp.init), up(inp.d_cum)
        del inp
        cum, d_q, d_init = torch.empty_like(q), torch.empty_like(q), torch.empty_like(init)
        fwd_bytes = 2 * io_bytes * n + io_bytes * cols
        bwd_bytes = 3 * io_bytes * n + 2 * io_bytes * cols
        for mode in ("saved boundary state", "final carry", "leaves-only"):
            ckpt = {"saved boundary state": lambda: capi.new_ckpt(q), "final carry": lambda: capi.new_ckpt(q, "final"),
                    "leaves-only": lambda: None}[mode]()

            def fwd():
                capi.quat_cumprod_fwd(q, init, cum, ckpt)

            def bwd():
                capi.quat_cumprod_bwd(q, init, d_cum, ckpt, d_q=d_q, d_init=d_init)

            warm, t0 = 0, time.perf_counter()
            while warm < args.warmup or (time.perf_counter() - t0) * 1e3 < args.settle_ms:
                fwd()
                bwd()
                warm += 1
                if warm % 16 == 0:
                    torch.cuda.synchronize()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                fwd()
                bwd()
            torch.cuda.synchronize()
            step_ms = (time.perf_counter() - t0) / args.steps * 1e3
            ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731
            diag = [((ev(), ev()), (ev(), ev())) for _ in range(20)]
            for (f0, f1), (b0, b1) in diag:
                f0.record()
                fwd()
                f1.record()
                b0.record()
                bwd()
                b1.record()
            torch.cuda.synchronize()
            if capi.default_workspace.status(dev) != 0:
                raise RuntimeError(f"{name}: a cross-block wait hit its spin limit")
            fwd_ms = float(np.median([a.elapsed_time(c) for (a, c), _ in diag]))
            bwd_ms = float(np.median([a.elapsed_time(c) for _, (a, c) in diag]))
            gb = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9   # noqa: E731
            rec = {
                "metric": "quat cumprod fwd+bwd GB/s and % HBM peak, per workload",
                "config": {"workload": f"{name}{'' if shards == 1 else f' shard 1/{shards}'} b{b} s{s} h{h} j{j} "
                                       f"{io} I/O, forward + backward", "b": b,
                           "s": s, "h": h, "j": j, "io_dtype": io, "recipe": recipe},
                "backward": mode, "steps": args.steps,
                "cache_resident": fwd_bytes < 256 * 2 ** 20,
                "step_us": round(step_ms * 1e3, 2), "fwd_us": round(fwd_ms * 1e3, 2),
                "bwd_us": round(bwd_ms * 1e3, 2),
                "GBps": round(gb(fwd_bytes + bwd_bytes, step_ms), 1),
                "fwd_GBps": round(gb(fwd_bytes, fwd_ms), 1), "bwd_GBps": round(gb(bwd_bytes, bwd_ms), 1),
                "hbm_frac": round(gb(fwd_bytes + bwd_bytes, step_ms) / HBM_PEAK_GBPS, 4),
                "fwd_hbm_frac": round(gb(fwd_bytes, fwd_ms) / HBM_PEAK_GBPS, 4),
                "bwd_hbm_frac": round(gb(bwd_bytes, bwd_ms) / HBM_PEAK_GBPS, 4),
                "elements_per_s": round(n / (step_ms * 1e-3), 1),
                "fwd_bytes": fwd_bytes, "bwd_bytes": bwd_bytes,
            }
            print(json.dumps(rec), flush=True)
        del q, init, d_cum, cum, d_q, d_init
        torch.cuda.empty_cache()


def short_kernel_name(name: str) -> str:
    for pre in ("void ", "qc::(anonymous namespace)::", "(anonymous namespace)::", "qc::"):
        name = name.replace(pre, "")
    return name.replace("(KernelArgs)", "")


def summarize_profile(trace_dir: str, config: str, pmc_dir: str | None, command: str, bench_log: str | None = None,
                      saved: str = "boundary", out_dir: str | None = None):
    """Write profiles/kernels_<config>.txt from a rocprofv3 --kernel-trace
    --stats run (and, with pmc_dir, its FETCH_SIZE / WRITE_SIZE runs scaled by
    the plain-copy calibration factors of traffic_headline.txt).  Kernel
    template arguments: forward <IO, column-group width, steps per lane,
    waves, stores cum, mode>, backward <IO, width, steps per lane, waves, mode,
    from the final carry>; mode 0 = Fenwick look-back, 3 = grouped look-back."""
    import csv
    import statistics

    from quaternion_cumprod_autodiff_amd.inputs import CONFIGS
    b, s, h, j, recipe, io = CONFIGS[config]
    rows = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))))
    mode = "saved boundary state" if saved == "boundary" else "backward from the final carry alone"
    lines = [f"# Kernel durations and HBM traffic, workload {config} (b{b} s{s} h{h} j{j}, {io} I/O, "
             f"recipe {recipe}, {mode}), one MI355X.",
             "# Commands (from /tmp, TMPDIR=/tmp, R = repository root, OUT = an output directory):"]
    lines += ["#   " + c for c in command.split(" ;; ")]
    lines.append("#")
    if bench_log:
        recs = [json.loads(x) for x in open(bench_log) if x.startswith("{")]
        if recs:
            d = recs[-1]
            lines.append(f"# The traced bench run's own line (profiler attached): {d['ms_per_step']} ms per step, "
                         f"{d['value']} GB/s ({d['hbm_frac']:.3f} of 8 TB/s); diagnostic fwd "
                         f"{d.get('diag_fwd_ms')} ms, bwd {d.get('diag_bwd_ms')} ms.")
            lines.append("#")
    lines.append("# rocprofv3 run_kernel_stats.csv (every dispatch of the traced run, untimed settle steps included)")
    lines.append(f"# {'kernel':70s} {'calls':>6s} {'avg ns':>10s} {'min ns':>10s} {'max ns':>10s}")
    for r in rows:
        name = short_kernel_name(r["Name"])
        lines.append(f"{name[:72]:72s} {int(r['Calls']):6d} {float(r['AverageNs']):10.0f} "
                     f"{float(r['MinNs']):10.0f} {float(r['MaxNs']):10.0f}")
    if pmc_dir:
        cal = read_kv(TRAFFIC_FILE)
        fs, ws = float(cal["fetch_scale"]), float(cal["write_scale"])

        def per_kernel(counter):
            vals = {}
            for r in csv.DictReader(open(os.path.join(pmc_dir, counter, "run_counter_collection.csv"))):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
            return {k: statistics.median(v) for k, v in vals.items()}

        f, w = per_kernel("FETCH_SIZE"), per_kernel("WRITE_SIZE")
        n, cols = b * s * h * j, b * h * j
        io_bytes = 16 if io == "f32" else 8
        alg = {"fwd_chunked_kernel": 2 * io_bytes * n + io_bytes * cols,
               "fwd_column_kernel": 2 * io_bytes * n + io_bytes * cols,
               "bwd_chunked_kernel": 3 * io_bytes * n + 2 * io_bytes * cols}
        lines.append("#")
        lines.append(f"# HBM bytes per launch: FETCH_SIZE x {fs:.4f} + WRITE_SIZE x {ws:.4f} (the plain-copy "
                     "calibration factors of traffic_headline.txt), median over the run's launches")
        lines.append(f"# {'kernel':70s} {'fetch B':>14s} {'write B':>14s} {'algorithmic B':>14s} {'ratio':>6s}")
        for k in sorted(set(f) & set(w)):
            if "zero_words" in k or "bump_epoch" in k or "at::native" in k or "rocclr" in k:
                continue
            # (no algorithmic share for the boundary pre-pass: a forward that stores no cum)
            prepass = re.search(r"fwd_chunked_kernel<.*, false, \d+>", k) is not None
            base = None if prepass else next((v for key, v in alg.items() if key in k), None)
            tot = f[k] * fs + w[k] * ws
            lines.append(f"{short_kernel_name(k)[:72]:72s} {f[k] * fs:14.0f} {w[k] * ws:14.0f} "
                         f"{(base if base else 0):14d} {(tot / base if base else 0):6.3f}")
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"),
                        f"kernels_{config}{'' if saved == 'boundary' else '_' + saved}.txt")
    with open(path, "w") as out:
        out.write("\n".join(lines) + "\n")
    print(path)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="keep running untimed warm-up steps until this much time has passed (the GPU's "
                         "clocks take tens of ms of sustained load to settle)")
    from quaternion_cumprod_autodiff_amd.inputs import CONFIGS, make_config
    ap.add_argument("--config", default="headline", choices=list(CONFIGS))
    ap.add_argument("--path", default=None, choices=["auto", "column", "chunked", "rscan"])
    ap.add_argument("--lookback", default=None, choices=["auto", "fenwick", "grouped"])
    ap.add_argument("--leaves", default=None, choices=["auto", "prepass", "coresident"],
                    help="how the leaves-only backward re-derives the boundary products")
    ap.add_argument("--saved", default="boundary", choices=["boundary", "final"],
                    help="what the timed forward saves for its backward (with --leaves-only: nothing)")
    ap.add_argument("--leaves-only", action="store_true",
                    help="backward without the saved boundary state (re-derives it from q)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time the steps without the backward's event records (each adds a few us of idle)")
    ap.add_argument("--leaves-steps", type=int, default=100,
                    help="after the timed region, also time this many steps of each other backward mode (0: skip)")
    ap.add_argument("--event-every", type=int, default=4,
                    help="bracket every N-th timed backward with events (N=1: every one)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only time a plain device copy of one [b,s,h,j,4] tensor")
    ap.add_argument("--summarize-traffic", metavar="PMC_DIR",
                    help="write profiles/traffic_headline.txt from rocprofv3 FETCH_SIZE/WRITE_SIZE runs")
    ap.add_argument("--scan", choices=["add", "quat"],
                    help="measure the generic scan VJP (include/qc_scan.h) with this body instead")
    ap.add_argument("--scan-k", type=int, default=0,
                    help="with --scan: VJP from k snapshots (binomial checkpointing); 0 = saved trajectory")
    ap.add_argument("--summarize-scan-traffic", metavar="PMC_DIR",
                    help="write profiles/traffic_scan_quat.txt from rocprofv3 runs of --scan quat")
    ap.add_argument("--gdn2", action="store_true",
                    help="measure the Gated DeltaNet-2 forward + VJP (include/gdn2.h) instead")
    ap.add_argument("--summarize-gdn2-traffic", metavar="PMC_DIR",
                    help="write profiles/traffic_gdn2.txt from rocprofv3 runs of --gdn2")
    ap.add_argument("--gdn2-chunk", type=int, default=0,
                    help="with --gdn2: steps between saved boundary states (default: the workload's)")
    ap.add_argument("--all-configs", action="store_true",
                    help="one JSON line per named workload and backward mode (forward, backward, step rates)")
    ap.add_argument("--seq-shards", type=int, default=1,
                    help="with --all-configs: time one GPU's share of a run sharded N ways along the sequence")
    ap.add_argument("--configs", default="",
                    help="with --all-configs: comma-separated workload names (default: all)")
    ap.add_argument("--summarize-profile", metavar="TRACE_DIR",
                    help="write profiles/kernels_<config>.txt from a rocprofv3 kernel-trace run of --config")
    ap.add_argument("--pmc-dir", default=None,
                    help="with --summarize-profile: directory holding FETCH_SIZE/ and WRITE_SIZE/ counter runs")
    ap.add_argument("--bench-log", default=None,
                    help="with --summarize-profile: the traced bench run's output, for its JSON line")
    ap.add_argument("--profile-command", default="",
                    help="with --summarize-profile: the commands that made the runs (' ;; '-separated)")
    args = ap.parse_args()
    if args.summarize_gdn2_traffic:
        B, H, T, L, D, C = GDN2_WORKLOAD
        summarize_gdn2_traffic(args.summarize_gdn2_traffic,
                               f"gdn2 b{B} h{H} t{T} latent{L} dense{D} chunk{C} f32, forward + VJP")
        return
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.config, args.pmc_dir, args.profile_command, args.bench_log,
                          args.saved)
        return
    if args.summarize_scan_traffic:
        cal = read_kv(TRAFFIC_FILE)
        summarize_scan_traffic(args.summarize_scan_traffic, float(cal["fetch_scale"]), float(cal["write_scale"]))
        return
    if args.summarize_traffic:
        b, s, h, j, _, io = CONFIGS["headline"]
        summarize_traffic(args.summarize_traffic, float(b * s * h * j * 16))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(columns shard across GPUs without communication)", file=sys.stderr)
        sys.exit(2)

    if args.scan:
        scan_bench(args)
        return
    if args.gdn2:
        gdn2_bench(args)
        return
    if args.all_configs:
        all_configs_bench(args)
        return

    import numpy as np
    import torch

    from quaternion_cumprod_autodiff_amd import capi

    b, s, h, j, recipe, io = CONFIGS[args.config]
    n = b * s * h * j
    cols = b * h * j
    io_bytes = 16 if io == "f32" else 8

    if args.copy_calibration:
        gbps, dt = copy_calibration(n * io_bytes, args.steps, args.warmup)
        print(json.dumps({"copy_bytes": n * io_bytes, "copy_GBps": round(gbps, 1), "ms": round(dt * 1e3, 4)}))
        return

    t0 = time.perf_counter()
    inp = make_config(args.config, want_f64=False)
    log(f"[bench] inputs {args.config} generated in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16 if io == "bf16" else np.float32)).to(dev)
        return t.view(torch.bfloat16) if io == "bf16" else t

    q, init, d_cum = up(inp.q), up(inp.init), up(inp.d_cum)
    cum = torch.empty_like(q)
    d_q = torch.empty_like(q)
    d_init = torch.empty_like(init)
    ckpt = None if args.leaves_only else capi.new_ckpt(q, args.saved)
    timed_mode = "leaves-only" if args.leaves_only else {"boundary": "saved boundary state",
                                                         "final": "final carry"}[args.saved]

    def fwd():
        capi.quat_cumprod_fwd(q, init, cum, ckpt, path=args.path, lookback=args.lookback)

    def bwd():
        capi.quat_cumprod_bwd(q, init, d_cum, ckpt, d_q=d_q, d_init=d_init, path=args.path, lookback=args.lookback,
                              leaves=args.leaves)

    # Untimed warm-up: W steps, continued until --settle-ms has passed.
    warm_steps, t0 = 0, time.perf_counter()
    while warm_steps < args.warmup or (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        fwd()
        bwd()
        warm_steps += 1
        if warm_steps % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    status = capi.default_workspace.status(dev)
    if status != 0:
        raise RuntimeError("a cross-block wait hit its spin limit during warm-up")

    # Timed region: K steps.  Events bracket every N-th backward (the dominant
    # kernel) on the stream it is launched on (the current stream); each event
    # pair leaves the GPU idle for a few us, so sampling keeps that cost out of
    # most steps while the average still covers launches across the region.
    ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731
    every = max(1, args.event_every)
    timed_k = [] if args.no_kernel_events else list(range(every - 1, args.steps, every))
    be = {k: (ev(), ev()) for k in timed_k}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        fwd()
        if k in be:
            be[k][0].record()
            bwd()
            be[k][1].record()
        else:
            bwd()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if capi.default_workspace.status(dev) != 0:
        raise RuntimeError("a cross-block wait hit its spin limit during the timed steps")
    bwd_ms = float(np.mean([a.elapsed_time(bb) for a, bb in be.values()])) if be else None

    # Diagnostics after the timed region: forward and backward each bracketed.
    diag = [((ev(), ev()), (ev(), ev())) for _ in range(20)]
    for (f0, f1), (b0, b1) in diag:
        f0.record()
        fwd()
        f1.record()
        b0.record()
        bwd()
        b1.record()
    torch.cuda.synchronize()
    fwd_ms = float(np.median([f0.elapsed_time(f1) for (f0, f1), _ in diag]))
    bwd_ms_diag = float(np.median([b0.elapsed_time(b1) for _, (b0, b1) in diag]))

    # The other backward modes, reported beside the timed one on the same
    # workload with the same algorithmic bytes: the page-faithful leaves-only
    # mode (the forward saves nothing beyond the leaves and the backward
    # re-derives the boundary state from q, one more read of q), and the
    # final-carry mode (the forward saves only cum[:, s-1]; the backward reads
    # q and d_cum once and rebuilds cum from the end of the sequence).
    def time_mode(state):
        def fwd_m():
            capi.quat_cumprod_fwd(q, init, cum, state, path=args.path, lookback=args.lookback)

        def bwd_m():
            capi.quat_cumprod_bwd(q, init, d_cum, state, d_q=d_q, d_init=d_init, path=args.path,
                                  lookback=args.lookback, leaves=args.leaves)

        # Its own settle phase: a mode timed right after a change of kernels
        # otherwise reads a few percent slow for its first tens of steps.
        warm, t_w = 0, time.perf_counter()
        while warm < 10 or (time.perf_counter() - t_w) * 1e3 < args.settle_ms / 2:
            fwd_m()
            bwd_m()
            warm += 1
            if warm % 16 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        t_m = time.perf_counter()
        for _ in range(args.leaves_steps):
            fwd_m()
            bwd_m()
        torch.cuda.synchronize()
        ms_m = (time.perf_counter() - t_m) / args.leaves_steps * 1e3
        if capi.default_workspace.status(dev) != 0:
            raise RuntimeError("a cross-block wait hit its spin limit during the extra steps")
        return ms_m

    other_modes = {}
    if args.leaves_steps > 0:
        if timed_mode != "final carry" and args.path != "rscan":   # (no final-carry reduce-then-scan)
            other_modes["final_carry"] = time_mode(capi.new_ckpt(q, "final"))
        if timed_mode != "leaves-only":
            other_modes["leaves_only"] = time_mode(None)

    ms_step = wall / args.steps * 1e3
    fwd_bytes = 2 * io_bytes * n + io_bytes * cols
    bwd_bytes = 3 * io_bytes * n + 2 * io_bytes * cols
    value = (fwd_bytes + bwd_bytes) / (ms_step * 1e-3) / 1e9
    # Roofline of the backward from its timed-region events (or, with
    # --no-kernel-events, from the diagnostic loop).
    bwd_ms_roof = bwd_ms if bwd_ms is not None else bwd_ms_diag
    bwd_gbps = bwd_bytes / (bwd_ms_roof * 1e-3) / 1e9
    workload = f"{args.config} b{b} s{s} h{h} j{j} {io} I/O, forward + backward"
    traffic = (load_traffic(workload) if (args.path in (None, "auto", "chunked") and args.lookback in (None, "auto")
                                          and timed_mode == "saved boundary state") else None)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64" if io == "f32" else "f32",
        "data": "synthetic",
        "config": {"workload": workload, "b": b, "s": s, "h": h, "j": j, "io_dtype": io, "recipe": recipe,
                   "path": args.path or "auto", "lookback": args.lookback or "auto",
                   "leaves": args.leaves or "auto", "backward": timed_mode},
        "hbm_frac": round(value / HBM_PEAK_GBPS, 4),
        "elements_per_s": round(n / (ms_step * 1e-3), 1),
        "untimed_steps": warm_steps,
        "bwd_ms": round(bwd_ms, 4) if bwd_ms is not None else None,
        "bwd_launches_timed": len(be),
        "diag_fwd_ms": round(fwd_ms, 4),
        "diag_bwd_ms": round(bwd_ms_diag, 4),
        "diag_fwd_GBps": round(fwd_bytes / (fwd_ms * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "kernel": "bwd_chunked_kernel", "achieved": round(bwd_gbps, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(bwd_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic},
        "cpu_baseline": None,
    }
    mode_text = {"leaves_only": "forward saves only q and init; backward re-derives the boundary state from q",
                 "final_carry": "forward saves only its final carry per column; backward reads q and d_cum once"}
    for key, ms_m in other_modes.items():
        rec[key] = {"value": round((fwd_bytes + bwd_bytes) / (ms_m * 1e-3) / 1e9, 2), "unit": "GB/s",
                    "hbm_frac": round((fwd_bytes + bwd_bytes) / (ms_m * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                    "ms_per_step": round(ms_m, 4), "steps": args.leaves_steps, "mode": mode_text[key]}
    # Practical ceiling beside the roofline: the library's hand-written
    # streaming copy of one tensor of the workload (read + write), after the
    # timed region, at its best grid of a short sweep.
    ceil = copy_ceiling(n * io_bytes)
    rec["copy_ceiling"] = ceil
    rec["roofline"]["frac_of_copy_ceiling"] = round(bwd_gbps / ceil["value"], 4)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        rec["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
