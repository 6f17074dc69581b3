#!/usr/bin/env python3
"""Benchmark of the bf16 TriMul forward on one MI355X.

Default workload: outgoing TriMul, B=1, N=4096, D=C=256, bf16 storage with
fp32 accumulation, z ~ N(0, 1), weights ~ N(0, 1/D), no mask (the shape the
fold-cp-ops README runs in its "Use" section).  One step is one trimul_fwd
call (LayerNorm+projection, contraction, LayerNorm+output) with every input
already resident in HBM.  Prints one JSON line on stdout.

FLOPs counted per call: 2*B*C*N^3 (contraction) + 2*B*N^2*D*(4C + D) (input
projections incl. the output gate) + 2*B*N^2*C*D (output projection).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TriMul fwd ms/call + TFLOP/s (% bf16 MFMA peak), B=1 N=4096 D=256"
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}   # MI355X dense matrix peaks (published)
PEAK_HBM_GBS = 8000.0
# HBM bytes per contraction launch, measured with rocprofv3 counters (see the
# file for the commands and the copy-kernel calibration); used only while the
# contraction kernel's sources are the ones the counters were taken on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k2_contract_hbm_traffic_out_bf16_b1_n4096_d256.json")
K2_SOURCES = [os.path.join(ROOT, "triangle_multiplication_amd", "csrc", f)
              for f in ("k2_contract.hip", "trimul_device.hpp")]


def k2_source_digest():
    h = hashlib.sha256()
    for f in K2_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(name, direction):
    """Counter-derived HBM bytes per contraction launch, or None if not taken on these sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("workload") != name or t.get("direction") != direction or t.get("sources_sha256") != k2_source_digest():
        return None
    return float(t["hbm_bytes_per_launch"])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _events_ms(fn, reps):
    import torch
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def cpu_baseline(wl, z, mask, w, direction, n_sample):
    """The fp64 oracle on a bounded sample, extrapolated linearly in work to the full call."""
    import oracle
    from triangle_multiplication_amd import inputs
    B, N, D, C = wl.B, wl.N, wl.D, wl.C
    I, J = inputs.sample_grid(N, n_sample, extra=wl.sample_extra())
    zA, mA, zB, mB, zG = oracle.gather_grid(z, mask, 0, I, J, direction)
    t0 = time.perf_counter()
    _, t = oracle.trimul_grid(N, w, zA, mA, zB, mB, zG, want_times=True)
    wall = time.perf_counter() - t0
    ni, nj = len(I), len(J)
    t_proj = t[0] * (B * N * N * 4 * C * D) / ((ni + nj) * N * 2 * C * D)
    t_con = t[1] * (B * N * N) / (ni * nj)
    t_out = t[2] * (B * N * N) / (ni * nj)
    total = t_proj + t_con + t_out
    return {
        "value": wl.flops() / total / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": ("%dx%d (i,j) output grid of batch 0 (%d+%d token rows projected, %d "
                   "contractions of length N); %.1f s of CPU work, stage times extrapolated "
                   "linearly in work to all B*N^2 outputs: %.0f s per call"
                   % (ni, nj, ni, nj, ni * nj, wall, total)),
        "extrapolated_s_per_call": total,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--direction", default=None)
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--cpu-sample", type=int, default=384,
                    help="side of the (i, j) grid the oracle computes for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-gib", type=int, default=0,
                    help="only run one plain device copy of this many GiB (counter calibration) and exit")
    ap.add_argument("--print-k2-digest", action="store_true",
                    help="print the digest of the contraction kernel's sources and exit")
    args = ap.parse_args()
    if args.print_k2_digest:
        print(k2_source_digest())
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs the single-GPU TriMul path only; --gpus %d (WORLD_SIZE=%d) is not "
              "supported: run with --gpus 1" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibration_copy_gib:
        n = args.calibration_copy_gib << 30
        src = torch.zeros(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copied %d bytes" % n)
        return
    from triangle_multiplication_amd import binding, inputs

    name = args.workload or inputs.HEADLINE
    wl = inputs.WORKLOADS[name]
    direction = args.direction or wl.directions[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("workload %s direction %s" % (name, direction))

    if wl.N <= 1024:
        z = inputs.make_z(wl.B, wl.N, wl.D, wl.dtype, var=wl.z_var, device="cpu").to(dev)
    else:
        z = inputs.make_z(wl.B, wl.N, wl.D, wl.dtype, var=wl.z_var, device=dev)
    tm = wl.token_mask()
    mask = None if tm is None else inputs.pair_mask(tm, wl.B, wl.dtype, device=dev)
    w = inputs.make_weights(wl.D, wl.C, wl.dtype)
    layer = binding.TriMul(w, wl.dtype)
    out = torch.empty_like(z)
    ws = layer.workspace(wl.B, wl.N, dev)
    fwd = lambda: binding.trimul_fwd(layer.h, z, mask, direction, out, ws)

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    log("warmup done")

    # Timed region: exactly `steps` forward calls, synchronised on both sides.
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(args.steps):
        fwd()
    e1.record(s)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    log("timed %d steps: %.3f ms/step (events %.3f)" % (args.steps, wall_ms, ev_ms))

    # Per-kernel durations: each stage entry point launches the same kernel
    # trimul_fwd launches, on the same stream, timed with events.
    B, N, D, C = wl.B, wl.N, wl.D, wl.C
    es = 2 if wl.dtype == "bf16" else 4
    NN = N * N
    ab_shape = binding.ab_storage_shape(wl.dtype, B, C, N)
    ab_bytes = es
    for n in ab_shape:
        ab_bytes *= n
    ab_slab = (ab_bytes + 255) // 256 * 256
    tdt = inputs.TORCH_DTYPES[wl.dtype]
    a_cm = ws[:ab_bytes].view(tdt).view(ab_shape)
    b_cm = ws[ab_slab:ab_slab + ab_bytes].view(tdt).view(ab_shape)
    o_cm = ws[2 * ab_slab:2 * ab_slab + B * C * NN * es].view(tdt).view(B, C, N, N)
    reps = args.kernel_reps
    k1_ms = _events_ms(lambda: binding.trimul_internal_project(layer.h, z, mask, direction, a_cm, b_cm), reps)
    k2_ms = _events_ms(lambda: binding.trimul_internal_contract(layer.h, a_cm, b_cm, o_cm), reps)
    k3_ms = _events_ms(lambda: binding.trimul_internal_output(layer.h, z, o_cm, out), reps)
    log("kernels: project %.3f ms, contract %.3f ms, output %.3f ms" % (k1_ms, k2_ms, k3_ms))

    flops = wl.flops()
    k2_flops = 2 * B * C * N ** 3
    k1_flops = 2 * B * NN * D * 4 * C
    k3_flops = 2 * B * NN * D * (D + C)
    k1_bytes = B * NN * (D * es + (es if mask is not None else 0) + 2 * C * es)
    k3_bytes = B * NN * (D * es + C * es + D * es)
    k2_bytes = 3 * B * C * NN * es
    peak = PEAK_TFLOPS[wl.dtype]
    k2_tf = k2_flops / (k2_ms * 1e-3) / 1e12
    value = flops / (wall_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": B, "N": N, "D": D, "C": C, "direction": direction,
                   "mask": wl.mask, "flops_per_call": flops},
        "pct_peak": round(100.0 * value / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(k2_tf, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(k2_tf / peak, 4), "traffic": measured_traffic(name, direction),
                     "kernel": "k2_contract",
                     "per_launch": "2*B*C*N^3 = %.4g FLOP" % k2_flops, "avg_ms": round(k2_ms, 4)},
        "kernels": {
            "k1_project": {"ms": round(k1_ms, 4), "tflops": round(k1_flops / k1_ms / 1e9, 2),
                           "hbm_gbs": round(k1_bytes / k1_ms / 1e6, 1),
                           "hbm_frac": round(k1_bytes / k1_ms / 1e6 / PEAK_HBM_GBS, 4)},
            "k2_contract": {"ms": round(k2_ms, 4), "tflops": round(k2_tf, 2),
                            "hbm_gbs": round(k2_bytes / k2_ms / 1e6, 1)},
            "k3_output": {"ms": round(k3_ms, 4), "tflops": round(k3_flops / k3_ms / 1e9, 2),
                          "hbm_gbs": round(k3_bytes / k3_ms / 1e6, 1),
                          "hbm_frac": round(k3_bytes / k3_ms / 1e6 / PEAK_HBM_GBS, 4)},
        },
        "ms_per_step_events": round(ev_ms, 4),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a sample) ...")
        result["cpu_baseline"] = cpu_baseline(wl, z, mask, w, direction, args.cpu_sample)
        log("cpu baseline done")
    else:
        result["cpu_baseline"] = None
    layer.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
