#!/usr/bin/env python3
"""Benchmark: encoded points/s of one forward + backward pass of the hash-grid encoding.

Default workload: 3D d-linear, L=16, F=2, T=2^19 rows per level, N 16..2048, 2^20 points
(the Instant-NGP standard size).  One step = zero the gradient buffer, forward (gamma),
backward (scatter-add into the tables) with inputs already resident in GPU memory.

Prints ONE JSON line.  Besides the headline value it carries
  roofline      achieved algorithmic GB/s of the dominant kernel against the 8 TB/s HBM peak,
                its average launch duration from HIP events on the launch stream, and the
                HBM traffic of one launch measured by rocprofv3 counters -- read from
                profiles/traffic_counters.json only when those counters were taken on
                kernel sources identical to the ones built now (else null);
  cpu_baseline  the plain CPU oracle timed on the host cores on a bounded sample.
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

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "encoded points/s fwd+bwd (3D L=16 T=2^19 F=2) + % of HBM roofline"
HEADLINE = "dlinear3d_L16_T19"

# Counter-measured traffic per entry-point call: written by --summarize-counters from two
# rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script, scaled by what the same
# counters read for the copy kernel's known traffic, and stamped with the digest of the
# kernel sources it was taken on.  A figure whose digest differs from the current sources
# is not reported.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
# kernels of each entry point (name fragments), for summing counters per call; the d-linear
# workloads run the counting pair, whose forward launches the count kernel
ENTRY_KERNELS = {
    "forward": ("forward", "pack_kernel", "levels_to_rows", "level_major_to_rows", "zero_columns"),
    "backward": ("count_kernel", "scan_", "plan_kernel", "scatter_kernel", "reduce_kernel", "upstream_levels",
                 "backward_kernel"),
}


def entry_kernels(workload: str) -> dict:
    if workload.startswith("dlinear"):
        return {"forward": ENTRY_KERNELS["forward"] + ("count_kernel",),
                "backward": tuple(f for f in ENTRY_KERNELS["backward"] if f != "count_kernel")}
    return ENTRY_KERNELS


def source_digest() -> str:
    """sha256 over the kernel and ABI sources (the library the counters were taken on)."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "multiresolution_hash_grid_multires_amd", "csrc")
    files = sorted(glob.glob(os.path.join(pkg, "*.hip")) + glob.glob(os.path.join(pkg, "*.h"))
                   + glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, entry: str):
    """(bytes per call, note) from the counter file when it matches the current sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no counter record"
    if rec.get("source_digest") != source_digest():
        return None, "counters were taken on other kernel sources"
    v = rec.get("workloads", {}).get(workload, {}).get(entry)
    return (int(v) if v is not None else None), ("profiles/traffic_counters.json" if v is not None
                                                  else "no counters for this workload")


def _counter_rows(run_dir: str, counter: str) -> dict:
    """{kernel name: [per-dispatch values]} from a rocprofv3 --pmc CSV under run_dir."""
    out: dict = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    if not out:
        raise SystemExit(f"no {counter} rows under {run_dir}")
    return out


def summarize_counters(args) -> int:
    """Turn four rocprofv3 --pmc runs (the workload's FETCH_SIZE and WRITE_SIZE, the copy
    calibration's FETCH_SIZE and WRITE_SIZE) into bytes per entry-point call, and record them
    in profiles/traffic_counters.json with the current source digest."""
    wl_fetch, wl_write, cp_fetch, cp_write = args.summarize_counters
    copy_bytes = args.copy_bytes or (1 << 30)
    kib = copy_bytes / 1024.0
    cf = _counter_rows(cp_fetch, "FETCH_SIZE")
    cw = _counter_rows(cp_write, "WRITE_SIZE")
    ck = next(k for k in cf if "copy_kernel" in k)
    f_factor = kib / (sum(cf[ck]) / len(cf[ck]))
    w_factor = kib / (sum(cw[ck]) / len(cw[ck]))
    fetch = _counter_rows(wl_fetch, "FETCH_SIZE")
    write = _counter_rows(wl_write, "WRITE_SIZE")
    calls = args.steps + args.warmup
    per_kernel, entries = {}, {"forward": 0.0, "backward": 0.0}
    for name, vals in fetch.items():
        entry = next((e for e, frags in entry_kernels(args.workload).items() if any(fr in name for fr in frags)),
                     None)
        if entry is None or "copy_kernel" in name:
            continue
        wv = write.get(name, [0.0])
        per_call = 1024.0 * (f_factor * sum(vals) + w_factor * sum(wv) * len(vals) / len(wv)) / calls
        per_kernel[name] = {"entry": entry, "dispatches_per_call": len(vals) / calls,
                            "fetch_KiB_per_dispatch": sum(vals) / len(vals),
                            "write_KiB_per_dispatch": sum(wv) / len(wv), "bytes_per_call": round(per_call)}
        entries[entry] += per_call
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    digest = source_digest()
    if rec.get("source_digest") != digest:
        rec = {"source_digest": digest, "workloads": {}, "kernels": {}}
    rec["calibration"] = {"copy_bytes": copy_bytes, "fetch_factor": round(f_factor, 4),
                          "write_factor": round(w_factor, 4)}
    rec["workloads"][args.workload] = {k: round(v) for k, v in entries.items()}
    rec["kernels"][args.workload] = per_kernel
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps({"workload": args.workload, **rec["workloads"][args.workload],
                      "calibration": rec["calibration"]}), flush=True)
    return 0


def algorithmic_bytes_per_point(spec: dict) -> dict:
    """Bytes the method itself moves per point: streamed inputs/outputs, every table value
    referenced (4 B per fp32 gather) and every fp32 atomic as a read-modify-write (8 B).
    With A of the L levels active (coarse-to-fine), the forward still writes full rows
    (zeros for the inactive levels) while gathers, upstream reads and scatters cover the A
    active levels."""
    d, L, F = spec["d"], spec["L"], spec["F"]
    A = int(spec.get("active_levels") or L)
    comps = 1 + d + (d if spec.get("d2_mode") == "diag" else 1) if spec["kind"] != "dlinear" else 1
    # table values referenced per point and level: the 2^d corners (Hermite: times the 2^d
    # coefficients of each); RBF: the (2k)^d vertices of the k-ring box
    corners = {"dlinear": 1 << d, "hermite": (1 << d) * (1 << d),
               "rbf": (2 * int(spec.get("rbf_rings") or 0)) ** d}[spec["kind"]]
    x_bytes = 4 * d
    return {"forward": x_bytes + 4 * L * F * comps + 4 * A * corners * F,
            "backward": x_bytes + 4 * A * F * comps + 8 * A * corners * F}


def copy_bandwidth(torch, api, nbytes: int = 4 << 30, steps: int = 10) -> float:
    """Achievable HBM bandwidth, read + write GB/s of the plain copy kernel over nbytes (16x
    the Infinity Cache, so the copy streams from HBM)."""
    n = nbytes // 4
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty(n, device="cuda:0")
    api.hashenc_diag_copy(src, dst)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        api.hashenc_diag_copy(src, dst)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    del src, dst
    return 8 * n / ms / 1e6


def copy_calibration(args, torch, api) -> int:
    """Plain streaming copy of --copy-bytes bytes: achievable bandwidth, and a launch of known
    traffic (read + write = 2 * bytes) against which memory counters are scaled."""
    n = args.copy_bytes // 4
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty(n, device="cuda:0")
    for _ in range(args.warmup):
        api.hashenc_diag_copy(src, dst)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        api.hashenc_diag_copy(src, dst)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    print(json.dumps({"copy_bytes": 4 * n, "ms": round(ms, 4), "read_plus_write_GBps": round(8 * n / ms / 1e6, 1)}),
          flush=True)
    return 0


def cache_read_calibration(args, torch, api) -> int:
    """L2-resident read of --cache-bytes bytes, --cache-reps passes per launch: the L2 read
    ceiling the gather kernels are set against (bytes read = cache bytes x reps)."""
    n = (args.cache_bytes // 4) // 32 * 32
    buf = torch.ones(n, device="cuda:0")
    out = torch.zeros(1, device="cuda:0")
    for _ in range(args.warmup):
        api.hashenc_diag_cache_read(buf, args.cache_reps, out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        api.hashenc_diag_cache_read(buf, args.cache_reps, out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    print(json.dumps({"cache_bytes": 4 * n, "reps": args.cache_reps, "ms": round(ms, 4),
                      "read_GBps": round(4 * n * args.cache_reps / ms / 1e6, 1)}), flush=True)
    return 0


def fill_calibration(args, torch) -> int:
    """Write-only bandwidth: torch's fill of --fill-bytes bytes (a buffer far larger than the
    Infinity Cache, so the writes reach HBM)."""
    buf = torch.empty(args.fill_bytes // 4, device="cuda:0")
    for _ in range(args.warmup):
        buf.fill_(1.0)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        buf.fill_(1.0)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    print(json.dumps({"fill_bytes": 4 * buf.numel(), "ms": round(ms, 4),
                      "write_GBps": round(4 * buf.numel() / ms / 1e6, 1)}), flush=True)
    return 0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def single_thread_rate(O, spec, x_h, params_h, ups_h, n_params, sec_per_point: float) -> dict:
    """The same oracle on one thread, over a prefix sized from the multi-thread rate to take
    about two seconds."""
    threads = O.max_threads()
    m = max(1, min(x_h.shape[0], int(2.0 / max(sec_per_point * threads, 1e-12))))
    O.set_threads(1)
    try:
        t0 = time.perf_counter()
        O.forward(spec, x_h[:m], params_h)
        O.backward(spec, x_h[:m], *[u[:m] for u in ups_h], n_params=n_params)
        dt = time.perf_counter() - t0
    finally:
        O.set_threads(threads)
    return {"value": round(m / dt, 1), "unit": "points/s", "cores": 1,
            "sample": f"the first {m} points of the same workload, one fwd+bwd", "seconds": round(dt, 2)}


def mlp_flops_per_point(d: int, n_in: int, hidden: int, depth: int) -> int:
    """Multiply-add FLOPs of the SIREN part per point: forward mode carries d + 2 rows
    (value, d gradients, Laplacian) through every layer; the reverse sweep costs one product
    for the weight gradients and one for the input adjoints per layer."""
    rows = d + 2
    fwd = 0
    for k in range(depth):
        fan_in = n_in if k == 0 else hidden
        fwd += 2 * rows * fan_in * hidden
    fwd += 2 * hidden  # output layer (Laplacian row)
    return 3 * fwd


def fd_mlp_flops_per_point(d: int, n_in: int, hidden: int, depth: int) -> int:
    """Multiply-add FLOPs of the SIREN part per point of the finite-difference comparator:
    2d+1 stencil points, each a value-only forward, and a reverse sweep costing twice the
    forward (weight gradients and input adjoints)."""
    fwd = 0
    for k in range(depth):
        fan_in = n_in if k == 0 else hidden
        fwd += 2 * fan_in * hidden
    fwd += 2 * hidden
    return (2 * d + 1) * 3 * fwd


def residual_bench(args, torch, api, I, W) -> int:
    """One fused residual step (hashenc_residual, Hermite) or one finite-difference comparator
    step (hashenc_fd_residual, d-linear, when the workload names an FD step)."""
    spec, m = W["spec"], dict(W["mlp"])
    if args.mlp_depth:
        m["depth"] = args.mlp_depth  # the pages' depth ablation (same width and omega)
    fd = "fd_eps" in W
    n = W["n_points"]
    dev = torch.device("cuda:0")
    enc = api.HashGridEncoding(spec)
    n_in = spec["L"] * spec["F"]
    d = spec["d"]
    mlp = api.Mlp(n_in, m["hidden"], m["depth"], m["omega"])
    x_h = I.points(W["id"], n, d, clustered_half=W.get("clustered_half", False))
    params_h = I.tables(W["id"], enc.n_params, W["tables"])
    mlp_h = I.siren_mlp(W["id"], n_in, m["hidden"], m["depth"])
    x = torch.from_numpy(x_h).to(dev)
    params = torch.from_numpy(params_h).to(dev)
    mlp_params = torch.from_numpy(mlp_h).to(dev)
    wsb = (api.hashenc_fd_residual_workspace_size(enc.handle, mlp, n) if fd
           else api.hashenc_residual_workspace_size(enc.handle, mlp, n))
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    r = torch.empty(n, device=dev)
    loss = torch.empty(1, device=dev)
    gp = torch.zeros(enc.n_params, device=dev)
    gm = torch.zeros(mlp_params.numel(), device=dev)

    def step():
        gp.zero_()
        gm.zero_()
        if fd:
            api.hashenc_fd_residual(enc.handle, mlp, W["fd_eps"], x, params, mlp_params, None, r, loss, gp, gm, ws)
        else:
            api.hashenc_residual(enc.handle, mlp, x, params, mlp_params, r, loss, gp, gm, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    if fd:
        # every stencil point: a d-linear forward and backward, plus the level-major encoder
        # rows and their upstream written and read once each
        alg = algorithmic_bytes_per_point(spec)
        active = int(spec.get("active_levels") or spec["L"])
        enc_bytes = (2 * d + 1) * (alg["forward"] + alg["backward"] + 4 * 4 * active * spec["F"]) * n
        flops = fd_mlp_flops_per_point(d, n_in, m["hidden"], m["depth"]) * n
    else:
        lap_spec = dict(spec, d2_mode="laplacian")  # active_levels carried over
        alg = algorithmic_bytes_per_point(lap_spec)
        enc_bytes = (alg["forward"] + alg["backward"]) * n
        flops = mlp_flops_per_point(d, n_in, m["hidden"], m["depth"]) * n

    cpu = None
    if not args.no_cpu_baseline:
        # the oracle as it stands on the host cores, on the first points of the same workload
        # (about --cpu-seconds of work), scaled to points/s
        from oracle import oracle as O
        k = 256
        while True:
            t0 = time.perf_counter()
            if fd:
                O.fd_residual(spec, m["hidden"], m["depth"], m["omega"], W["fd_eps"], x_h[:k], params_h, mlp_h)
            else:
                O.residual(spec, m["hidden"], m["depth"], m["omega"], x_h[:k], params_h, mlp_h)
            dt = time.perf_counter() - t0
            if dt > 0.3 * args.cpu_seconds or k >= n:
                break
            k = min(n, int(k * min(16.0, max(2.0, 0.5 * args.cpu_seconds / max(dt, 1e-3)))))
        cpu = {"value": round(k / dt, 1), "unit": "points/s", "cores": O.max_threads(), "kind": "oracle",
               "sample": f"the first {k} of the {n} points of the same workload, one step (fp64 oracle)",
               "seconds": round(dt, 2), "cpu_model": cpu_model()}

    what = "INGP-FD comparator steps" if fd else "PINN residual steps"
    print(json.dumps({
        "metric": f"{what}: points/s ({args.workload}"
                  + (f", {args.active_levels} of {spec['L']} levels active)" if args.active_levels else ")"),
        "value": round(n / (ms * 1e-3), 1),
        "unit": "points/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "n_points": n, "hidden": m["hidden"], "depth": m["depth"],
                   "omega": m["omega"], "active_levels": int(spec.get("active_levels") or spec["L"]),
                   **({"fd_eps": W["fd_eps"]} if fd else {})},
        "encoder_alg_GBps_over_step": round(enc_bytes / (ms * 1e-3) / 1e9, 1),
        "mlp_TFLOPs_over_step": round(flops / (ms * 1e-3) / 1e12, 2),
        "cpu_baseline": cpu,
        "loss": float(loss.item())}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--backward", choices=["binned", "atomic"], default="binned",
                    help="binned: hashenc_forward_ws + hashenc_backward_ws (workspace); "
                         "atomic: hashenc_forward + hashenc_backward (no workspace)")
    ap.add_argument("--active-levels", type=int, default=0,
                    help="coarse-to-fine activation: compute only the first A levels (0: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-counting", action="store_true",
                    help="d-linear: hashenc_forward_ws + hashenc_backward_ws instead of the counting pair")
    ap.add_argument("--mlp-depth", type=int, default=0,
                    help="residual workloads: SIREN hidden layers instead of the workload's own (1..4)")
    ap.add_argument("--n-points", type=int, default=0,
                    help="points per step instead of the workload's own count (the first N of its points)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the benchmark, run the plain copy kernel over this many bytes "
                         "(bandwidth and memory-counter calibration)")
    ap.add_argument("--cache-bytes", type=int, default=0,
                    help="instead of the benchmark, read this many bytes (split over the 8 XCDs' L2s) "
                         "--cache-reps times per launch: the L2 read ceiling")
    ap.add_argument("--cache-reps", type=int, default=200)
    ap.add_argument("--fill-bytes", type=int, default=0,
                    help="instead of the benchmark, time torch's fill of this many bytes (write-only bandwidth)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("WL_FETCH", "WL_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="instead of the benchmark, turn the output folders of four rocprofv3 --pmc runs "
                         "(this workload's FETCH_SIZE and WRITE_SIZE runs with the same --steps/--warmup, "
                         "the copy calibration's FETCH_SIZE and WRITE_SIZE runs with the same --copy-bytes) "
                         "into bytes per entry-point call in profiles/traffic_counters.json")
    args = ap.parse_args()
    if args.summarize_counters:
        return summarize_counters(args)
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (--gpus {args.gpus} requested); "
              "the multi-GPU sharding is a design, not a measured path", file=sys.stderr)
        return 2

    import torch

    from multiresolution_hash_grid_multires_amd import api
    from multiresolution_hash_grid_multires_amd import inputs as I

    if args.copy_bytes:
        return copy_calibration(args, torch, api)
    if args.cache_bytes:
        return cache_read_calibration(args, torch, api)
    if args.fill_bytes:
        return fill_calibration(args, torch)

    W = I.WORKLOADS[args.workload]
    if args.n_points:
        W = dict(W, n_points=args.n_points)
    if args.active_levels:
        W = dict(W, spec=dict(W["spec"], active_levels=args.active_levels))
    if "mlp" in W:
        return residual_bench(args, torch, api, I, W)
    spec = W["spec"]
    n = W["n_points"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    enc = api.HashGridEncoding(spec)
    x_h = I.workload_points(args.workload)[:n] if "stratified_side" in W else I.points(W["id"], n, spec["d"])
    params_h = I.tables(W["id"], enc.n_params, W["tables"])
    shapes = enc.output_shapes(n)
    ups_h = I.upstream(W["id"], list(shapes.values()))
    x = torch.from_numpy(x_h).to(dev)
    params = torch.from_numpy(params_h).to(dev)
    outs = {k: torch.empty(s, device=dev) for k, s in shapes.items()}
    ups = [torch.from_numpy(u).to(dev) for u in ups_h]
    ups += [None] * (3 - len(ups))
    grad = torch.zeros(enc.n_params, device=dev)
    stream = torch.cuda.current_stream()
    workspace = enc.workspace(n) if args.backward == "binned" else None
    # the backward the library actually runs: the workspace entry point falls back to the
    # atomic scatter-add when the configuration has no binned plan (RBF; 4D Hermite with F = 8)
    backward_path = ("binned" if workspace is not None and api.hashenc_backward_workspace_size(enc.handle, n) > 0
                     else "atomic")
    # d-linear: the counting pair (the forward takes the backward's bin counts while it
    # gathers; separate forward and backward workspaces)
    counting = workspace is not None and spec["kind"] == "dlinear" and not args.no_counting
    if counting:
        fws, bws = enc.forward_workspace(n), enc.backward_workspace(n)
        if backward_path == "binned":
            backward_path = "binned, counts taken by the forward"

    def step(ev=None):
        if ev is not None:
            ev[3].record(stream)
        grad.zero_()
        if ev is not None:
            ev[0].record(stream)
        if counting:
            api.hashenc_forward_counting(enc.handle, x, params, outs["gamma"], None, None, fws, bws)
        elif workspace is not None:
            api.hashenc_forward_ws(enc.handle, x, params, outs["gamma"], outs.get("dgamma"), outs.get("d2gamma"),
                                   workspace)
        else:
            api.hashenc_forward(enc.handle, x, params, outs["gamma"], outs.get("dgamma"), outs.get("d2gamma"))
        if ev is not None:
            ev[1].record(stream)
        if counting:
            api.hashenc_backward_counted(enc.handle, x, ups[0], None, None, grad, bws)
        elif workspace is not None:
            api.hashenc_backward_ws(enc.handle, x, ups[0], ups[1], ups[2], grad, workspace)
        else:
            api.hashenc_backward(enc.handle, x, ups[0], ups[1], ups[2], grad)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, HIP events on the launch stream around each kernel
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        step(evs[k])
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    step_median_ms = float(np.median([e[3].elapsed_time(e[2]) for e in evs]))
    ms_per_step = total_ms / args.steps
    value = n / (ms_per_step * 1e-3)

    alg = algorithmic_bytes_per_point(spec)
    kern = {"forward": {"ms": fwd_ms, "alg_bytes": alg["forward"] * n},
            "backward": {"ms": bwd_ms, "alg_bytes": alg["backward"] * n}}
    for k in kern.values():
        k["GBps"] = k["alg_bytes"] / (k["ms"] * 1e-3) / 1e9
    dom = max(kern, key=lambda k: kern[k]["ms"])
    # counters are recorded for the default (workspace) entry points with every level active
    traffic, traffic_note = ((recorded_traffic(args.workload, dom)) if workspace is not None and not args.active_levels
                             else (None, "counters recorded for the workspace entry points, all levels active"))
    roofline = {"bound": "hbm", "achieved": round(kern[dom]["GBps"], 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(kern[dom]["GBps"] / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "traffic_source": traffic_note, "source_digest": source_digest(),
                "kernel": ("hashenc_" + dom + (("_counting" if dom == "forward" else "_counted") if counting
                                                else "_ws" if workspace is not None else "")
                           + f" ({spec['kind']}; its kernels back to back on one stream)"),
                "avg_launch_ms": round(kern[dom]["ms"], 4),
                "alg_bytes_per_launch": kern[dom]["alg_bytes"]}
    # the same launch against the copy kernel's bandwidth measured now (read + write), and the
    # counter-measured traffic of the launch as a bandwidth
    achievable = copy_bandwidth(torch, api)
    roofline["achievable_GBps"] = round(achievable, 1)
    roofline["frac_of_achievable"] = round(kern[dom]["GBps"] / achievable, 4)
    if traffic is not None:
        roofline["traffic_GBps"] = round(traffic / (kern[dom]["ms"] * 1e-3) / 1e9, 1)
    step_alg = alg["forward"] + alg["backward"]

    cpu = None
    if not args.no_cpu_baseline:
        # the oracle as it stands, on the host cores: a prefix of the same points, grown until
        # one fwd+bwd takes a fair share of --cpu-seconds; if the whole workload is that fast,
        # it is repeated to fill about --cpu-seconds
        from oracle import oracle as O
        m = min(n, 1 << 16)
        for _ in range(8):
            xs = x_h[:m]
            us = [u[:m] for u in ups_h]
            t0 = time.perf_counter()
            O.forward(spec, xs, params_h)
            O.backward(spec, xs, *us, n_params=enc.n_params)
            dt = time.perf_counter() - t0
            if dt > 0.2 * args.cpu_seconds or m == n:
                break
            m = min(n, int(m * min(16.0, max(2.0, 0.3 * args.cpu_seconds / max(dt, 1e-3)))))
        reps, total = 1, dt
        if m == n and dt < args.cpu_seconds:
            reps = max(1, int(args.cpu_seconds / max(dt, 1e-3)))
            t0 = time.perf_counter()
            for _ in range(reps):
                O.forward(spec, x_h, params_h)
                O.backward(spec, x_h, *ups_h, n_params=enc.n_params)
            total = time.perf_counter() - t0
        what = (f"all {n} points of the same workload, one fwd+bwd, repeated {reps} times" if m == n
                else f"the first {m} of the {n} points of the same workload, one fwd+bwd")
        cpu = {"value": round(reps * m / total, 1), "unit": "points/s", "cores": O.max_threads(),
               "kind": "oracle", "sample": what + " (fp64-accumulating oracle, not a tuned CPU encoder)",
               "seconds": round(total, 2), "cpu_model": cpu_model(),
               "single_thread": single_thread_rate(O, spec, x_h, params_h, ups_h, enc.n_params, total / reps / m)}

    metric = (METRIC if args.workload == HEADLINE and not args.n_points
              else f"encoded points/s fwd+bwd ({args.workload}" + (f", {n} points)" if args.n_points else ")"))
    if args.active_levels:
        metric = f"encoded points/s fwd+bwd ({args.workload}, {args.active_levels} of {spec['L']} levels active)"
    line = {
        "metric": metric,
        "value": round(value, 1),
        "unit": "points/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "n_points": n, "d": spec["d"], "L": spec["L"],
                   "F": spec["F"], "T": spec["T"], "kind": spec["kind"], "backward": backward_path,
                   "active_levels": int(spec.get("active_levels") or spec["L"])},
        "ms_per_step_median": round(step_median_ms, 4),
        "hbm_roofline_pct_step": round(100.0 * value * step_alg / (HBM_PEAK_GBPS * 1e9), 2),
        "kernels": {k: {"ms": round(v["ms"], 4), "GBps": round(v["GBps"], 1)} for k, v in kern.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
