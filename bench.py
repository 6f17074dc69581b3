#!/usr/bin/env python3
"""Benchmark of the bf16 TriMul forward on one MI355X.

Default workload: outgoing TriMul, B=1, N=4096, D=C=256, bf16 storage with
fp32 accumulation, z ~ N(0, 1), weights ~ N(0, 1/D), no mask (the shape the
fold-cp-ops README runs in its "Use" section).  One step is one trimul_fwd
call (LayerNorm+projection, contraction, LayerNorm+output; on masked
workloads also the mask scan) with every input already resident in HBM.
Prints one JSON line on stdout.

FLOPs counted per call: 2*B*C*N^3 (contraction) + 2*B*N^2*D*(4C + D) (input
projections incl. the output gate) + 2*B*N^2*C*D (output projection).
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HEADLINE_METRIC = "TriMul fwd ms/call + TFLOP/s (% bf16 MFMA peak), B=1 N=4096 D=256"
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}   # MI355X dense matrix peaks (published)
PEAK_HBM_GBS = 8000.0
# HBM bytes per contraction launch, measured with rocprofv3 counters (see the
# file for the commands and the copy-kernel calibration); used only while the
# contraction kernel's sources are the ones the counters were taken on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k2_contract_hbm_traffic_out_bf16_b1_n4096_d256.json")
K2_SOURCES = [os.path.join(ROOT, "triangle_multiplication_amd", "csrc", f)
              for f in ("k2_contract.hip", "trimul_device.hpp")]
FLUSH_BYTES = 512 << 20   # larger than the last-level cache (256 MB)


def k2_source_digest():
    h = hashlib.sha256()
    for f in K2_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(name, direction, plan):
    """Counter-derived HBM bytes per contraction launch, or None unless the
    stored figure was taken on these sources, this workload and this plan."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if (t.get("workload") != name or t.get("direction") != direction
            or t.get("sources_sha256") != k2_source_digest()
            or tuple(t.get("plan", (0, 0, 8, 256))[1:]) != tuple(plan[1:])):
        return None
    return float(t["hbm_bytes_per_launch"])


def metric_for(wl, headline):
    if wl.name == headline:
        return HEADLINE_METRIC
    m = "TriMul fwd ms/call + TFLOP/s (%% %s MFMA peak), B=%d N=%d D=%d" % (wl.dtype, wl.B, wl.N, wl.D)
    return m if wl.C == wl.D else m + " C=%d" % wl.C


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


def host_facts():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return model, nproc


def _omp_set_threads(n):
    """Set the OpenMP thread count of this thread's later parallel regions."""
    import ctypes
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
        return True
    except OSError:
        return False


def cpu_baseline(wl, z, mask, w, direction, n_sample):
    """The fp64 oracle as it stands, on the host cores: in full for N <= 512
    (also on one thread), else on a bounded (i, j) grid with each stage's time
    extrapolated linearly in work to the full call."""
    import numpy as np
    import oracle
    from triangle_multiplication_amd import inputs
    B, N, D, C = wl.B, wl.N, wl.D, wl.C
    model, nproc = host_facts()
    threads = oracle.max_threads()
    res = {"unit": "TFLOP/s", "cores": threads, "nproc": nproc, "cpu_model": model, "kind": "oracle"}
    if N <= 512:
        zf = z.float().cpu().numpy()
        mf = None if mask is None else mask.float().cpu().numpy()

        def per_call():
            # whole calls, repeated until they add up to at least 2 s; the mean
            n, t0 = 0, time.perf_counter()
            while True:
                oracle.trimul_full(zf, mf, w, direction)
                n += 1
                t = time.perf_counter() - t0
                if t >= 2.0:
                    return t / n, n

        t_all, reps = per_call()
        res.update(value=wl.flops() / t_all / 1e12, seconds_per_call=t_all,
                   sample="the whole call (all B*N^2 outputs), mean of %d calls: %.4g s per call on %d threads"
                          % (reps, t_all, threads))
        if _omp_set_threads(1):
            t_one, reps1 = per_call()
            _omp_set_threads(threads)
            res.update(value_1thread=wl.flops() / t_one / 1e12, seconds_per_call_1thread=t_one,
                       calls_1thread=reps1)
        return res
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
    res.update(value=wl.flops() / total / 1e12, extrapolated_s_per_call=total,
               sample=("%dx%d (i,j) output grid of batch 0 (%d+%d token rows projected, %d "
                       "contractions of length N); %.1f s of CPU work, stage times extrapolated "
                       "linearly in work to all B*N^2 outputs: %.0f s per call"
                       % (ni, nj, ni, nj, ni * nj, wall, total)))
    return res


def measure_peaks(binding, torch, dev, reps=5):
    """What the chip delivers to the simplest code on this machine: the bf16 rate
    of an MFMA-only loop (two waves per SIMD, operands in registers, random
    data) and the HBM rate of plain 16-byte streams with the kernels' read and
    write mixes (1 GiB per buffer).  Best of `reps` timed launches each."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    g = torch.Generator(device="cpu").manual_seed(5)
    seed = torch.randn(2048, generator=g).to(torch.bfloat16).to(dev)
    blocks, iters = 2 * cus, 8192
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    mfma_flops = 4 * 262144 * iters * blocks
    shape_tf = {}
    for _ in range(2):          # warm both shapes up first (the clock ramps over the first launches)
        for shape in (0, 1):
            _events_ms(lambda: binding.trimul_internal_peak_mfma(seed, blocks, iters, sink, shape=shape), 1)
    for shape, key in ((0, "16x16x32"), (1, "32x32x16")):
        ms = min(_events_ms(lambda: binding.trimul_internal_peak_mfma(seed, blocks, iters, sink, shape=shape), 1)
                 for _ in range(reps))
        shape_tf[key] = round(mfma_flops / (ms * 1e-3) / 1e12, 1)
    mfma_tf = max(shape_tf.values())
    n = 1 << 30
    bufs = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(4)]
    for b in bufs[:2]:
        b.fill_(7)
    s0, s1, d0, d1 = bufs
    rates = {}
    for key, nbytes, kw in (("copy", 2 * n, {}), ("read2_write1", 3 * n, {"src1": s1}),
                            ("read1_write2", 3 * n, {"dst1": d1})):
        best = None
        for nt in (False, True):
            fn = lambda: binding.trimul_internal_peak_stream(s0, d0, nontemporal=nt, **kw)   # noqa: E731
            _events_ms(fn, 1)
            ms = min(_events_ms(fn, 1) for _ in range(reps))
            best = ms if best is None else min(best, ms)
        rates[key] = round(nbytes / best / 1e6, 1)
    del bufs, s0, s1, d0, d1
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(mfma_tf, 1), "mfma_bf16_tflops_by_shape": shape_tf, "stream_gbs": rates,
            "method": ("MFMA-only loop: %d workgroups x 4 waves x %d iterations of 16 independent "
                       "16x16x32 (or 8 32x32x16) bf16 MFMAs on register operands, the faster shape kept; streams: one 16-byte chunk per thread over "
                       "1 GiB buffers (copy: 1 read 1 write; read2_write1: the output stage's mix; "
                       "read1_write2: the projection's), plain and non-temporal, the faster kept; best of %d "
                       "launches, HIP events" % (blocks, iters, reps))}


def executed_k2_flops(table, B, C, N, tile=256):
    """FLOPs the masked contraction executes: per tile pair, 2 * tile^2 *
    (8192 / tile) per live key step of 8192 / tile keys (dead tiles run one
    step of zeros, not counted).  The table's ranges are in 32-key blocks of
    256-row tiles; a 128-row tile takes the range of the 256-row tile holding
    it, widened to whole 64-key steps."""
    import numpy as np
    from triangle_multiplication_amd import binding
    r = binding.table_parts(table, B, N)[0].cpu().numpy()
    kh = 256 // tile
    nt = (N + tile - 1) // tile
    tot = 0
    for b in range(r.shape[0]):
        u = np.arange(nt) * tile // 256
        lo, hi = r[b, u, 0], r[b, u, 1]
        L = np.maximum(lo[:, None], lo[None, :])
        H = np.minimum(hi[:, None], hi[None, :])
        live = H > L
        tot += int(np.where(live, (H + kh - 1) // kh - L // kh, 0).sum())
    return 2 * tile * tile * 32 * kh * C * tot


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--shape", default=None, metavar="B,N,D,C",
                    help="time a synthetic bf16 shape (no mask, z ~ N(0,1), outgoing unless --direction) "
                         "instead of a named workload")
    ap.add_argument("--direction", default=None, choices=[None, "outgoing", "incoming", "both"],
                    help="'both' runs the two directions in every step, in an order rotated per step")
    ap.add_argument("--cold", default="auto", choices=["auto", "on", "off"],
                    help="flush the caches (512 MiB write) before every timed call and time each call "
                         "with its own events; auto = on for N <= 1024")
    ap.add_argument("--tune", action="store_true", help="run trimul_tune first and time the tuned plan")
    ap.add_argument("--lean", action="store_true", help="use the workspace-lean layout")
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--cpu-sample", type=int, default=384,
                    help="side of the (i, j) grid the oracle computes for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-measured-peaks", action="store_true",
                    help="skip the MFMA-only and stream kernels that measure this box's ceilings")
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

    if args.shape:
        try:
            sB, sN, sD, sC = (int(x) for x in args.shape.split(","))
        except ValueError:
            print("--shape takes four integers B,N,D,C; got %r" % args.shape, file=sys.stderr)
            sys.exit(2)
        name = "shape_bf16_b%d_n%d_d%d_c%d" % (sB, sN, sD, sC)
        wl = inputs.Workload(name, "bf16", ("outgoing",), sB, sN, sD, sC, check="grid")
    else:
        name = args.workload or inputs.HEADLINE
        wl = inputs.WORKLOADS[name]
    if args.direction == "both":
        directions = ["outgoing", "incoming"]
    else:
        directions = [args.direction or wl.directions[0]]
    cold = args.cold == "on" or (args.cold == "auto" and wl.N <= 1024)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("workload %s directions %s cold %s" % (name, directions, cold))

    if wl.N <= 1024:
        z = inputs.make_z(wl.B, wl.N, wl.D, wl.dtype, var=wl.z_var, device="cpu").to(dev)
    else:
        z = inputs.make_z(wl.B, wl.N, wl.D, wl.dtype, var=wl.z_var, device=dev)
    tm = wl.token_mask()
    mask = None if tm is None else inputs.pair_mask(tm, wl.B, wl.dtype, device=dev)
    w = inputs.make_weights(wl.D, wl.C, wl.dtype)
    layer = binding.TriMul(w, wl.dtype)
    B, N, D, C = wl.B, wl.N, wl.D, wl.C
    out = torch.empty_like(z)
    if args.lean:
        ws = torch.empty(binding.trimul_workspace_size_lean(layer.h, B, N), dtype=torch.uint8, device=dev)
    else:
        ws = layer.workspace(B, N, dev)
    if args.tune:
        for d in directions:
            t0 = time.perf_counter()
            binding.trimul_tune(layer.h, z, mask, d, out, ws)
            log("tuned %s in %.2f s: plan %s" % (d, time.perf_counter() - t0,
                                                  binding.trimul_internal_get_plan(layer.h, B, N, d, mask is not None)))
    plans = {d: binding.trimul_internal_get_plan(layer.h, B, N, d, mask is not None) for d in directions}
    fwd = {d: (lambda d=d: binding.trimul_fwd(layer.h, z, mask, d, out, ws)) for d in directions}
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev) if cold else None

    for _ in range(args.warmup):
        for d in directions:
            fwd[d]()
    torch.cuda.synchronize()
    log("warmup done")

    # Timed region: exactly `steps` steps (one call per direction, the order
    # rotated per step), synchronised on both sides.  Cold: a cache flush
    # before every call, each call timed by its own events.
    s = torch.cuda.current_stream()
    per_call = {d: [] for d in directions}
    ev = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(s)
    for k in range(args.steps):
        order = directions[k % len(directions):] + directions[:k % len(directions)]
        for d in order:
            if cold:
                flush.zero_()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(s)
                fwd[d]()
                b.record(s)
                ev.append((d, a, b))
            else:
                fwd[d]()
    e1.record(s)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    for d, a, b in ev:
        per_call[d].append(a.elapsed_time(b))
    if cold:
        # A step's GPU time without the flushes: the per-call medians summed.
        step_ms = sum(statistics.median(per_call[d]) for d in directions)
        timing = ("per-call HIP events with the caches flushed (512 MiB write) before every call; "
                  "ms_per_step = sum over directions of the median call")
    else:
        step_ms = wall_ms
        timing = "wall clock over the timed steps, synchronised on both sides"
    log("timed %d steps: %.3f ms/step (wall %.3f, events %.3f)" % (args.steps, step_ms, wall_ms, ev_ms))

    # Per-kernel durations: each stage entry point launches the same kernel
    # trimul_fwd launches, on the same stream, timed with events (first
    # direction; masked workloads time the mask scan and the skipping
    # contraction, as trimul_fwd runs them).
    direction = directions[0]
    es = 2 if wl.dtype == "bf16" else 4
    NN = N * N
    tdt = inputs.TORCH_DTYPES[wl.dtype]
    ab_shape = binding.ab_storage_shape(wl.dtype, B, C, N)
    a_cm = torch.empty(ab_shape, dtype=tdt, device=dev) if args.lean else None
    if args.lean:
        b_cm = torch.empty_like(a_cm)
        o_cm = torch.empty((B, C, N, N), dtype=tdt, device=dev)
        rng = torch.empty(binding.mask_table_ints(B, N), dtype=torch.int32, device=dev)
    else:
        ab_bytes = es
        for n in ab_shape:
            ab_bytes *= n
        ab_slab = (ab_bytes + 255) // 256 * 256
        o_bytes = (B * C * NN * es + 255) // 256 * 256
        a_cm = ws[:ab_bytes].view(tdt).view(ab_shape)
        b_cm = ws[ab_slab:ab_slab + ab_bytes].view(tdt).view(ab_shape)
        o_cm = ws[2 * ab_slab:2 * ab_slab + B * C * NN * es].view(tdt).view(B, C, N, N)
        roff = 2 * ab_slab + o_bytes
        rng = ws[roff:roff + 4 * binding.mask_table_ints(B, N)].view(torch.int32)
    use_ranges = mask is not None and wl.dtype == "bf16"
    reps = args.kernel_reps
    k0_ms = None
    if use_ranges:
        k0_ms = _events_ms(lambda: binding.trimul_internal_mask_ranges(layer.h, mask, direction, rng), reps)
    k1_ms = _events_ms(lambda: binding.trimul_internal_project(layer.h, z, mask, direction, a_cm, b_cm), reps)
    rarg = rng if use_ranges else None
    k2_ms = _events_ms(lambda: binding.trimul_internal_contract(layer.h, a_cm, b_cm, o_cm, rarg, direction), reps)
    k3_ms = _events_ms(lambda: binding.trimul_internal_output(layer.h, z, o_cm, out), reps)
    log("kernels: mask scan %s ms, project %.3f ms, contract %.3f ms, output %.3f ms"
        % ("-" if k0_ms is None else "%.3f" % k0_ms, k1_ms, k2_ms, k3_ms))

    flops = wl.flops() * len(directions)
    k2_flops = 2 * B * C * N ** 3
    k1_flops = 2 * B * NN * D * 4 * C
    k3_flops = 2 * B * NN * D * (D + C)
    k1_bytes = B * NN * (D * es + (es if mask is not None else 0) + 2 * C * es)
    k3_bytes = B * NN * (D * es + C * es + D * es)
    k2_bytes = 3 * B * C * NN * es
    peak = PEAK_TFLOPS[wl.dtype]
    k2_tf = k2_flops / (k2_ms * 1e-3) / 1e12
    value = flops / (step_ms * 1e-3) / 1e12
    plan = plans[direction]
    traffic = stored_traffic(name, direction, plan) if not use_ranges else None
    roof = {"bound": "mfma", "achieved": round(k2_tf, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(k2_tf / peak, 4), "traffic": traffic,
            "traffic_source": ("stored counter figure: rocprofv3 FETCH_SIZE + WRITE_SIZE of this kernel "
                               "build, copy-calibrated, from %s (null when the contraction sources, "
                               "workload or plan differ)" % os.path.relpath(TRAFFIC_FILE, ROOT)),
            "kernel": "k2_contract",
            "per_launch": "2*B*C*N^3 = %.4g FLOP" % k2_flops, "avg_ms": round(k2_ms, 4),
            "plan": {"k1_variant": plan[0], "k2_order": plan[1], "k2_gm": plan[2], "k2_tile": plan[3]}}
    if use_ranges:
        ex = executed_k2_flops(rng, B, C, N, plan[3])
        roof["executed_flops_per_launch"] = ex
        roof["executed_tflops"] = round(ex / (k2_ms * 1e-3) / 1e12, 2)
    result = {
        "metric": metric_for(wl, inputs.HEADLINE), "value": round(value, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": B, "N": N, "D": D, "C": C, "directions": directions,
                   "mask": wl.mask, "flops_per_call": wl.flops(), "lean_workspace": bool(args.lean),
                   "tuned": bool(args.tune)},
        "timing": timing,
        "pct_peak": round(100.0 * value / peak, 2),
        "roofline": roof,
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
        "ms_per_step_wall": round(wall_ms, 4),
        "ms_per_step_events": round(ev_ms, 4),
    }
    if not args.no_measured_peaks and wl.dtype == "bf16":
        log("measured peaks ...")
        mp = measure_peaks(binding, torch, dev)
        result["measured_peaks"] = mp
        sg = mp["stream_gbs"]
        roof["measured_peak"] = mp["mfma_bf16_tflops"]
        roof["frac_measured"] = round(k2_tf / mp["mfma_bf16_tflops"], 4)
        kk = result["kernels"]
        kk["k2_contract"]["mfma_frac_measured"] = roof["frac_measured"]
        kk["k1_project"]["hbm_frac_measured"] = round(kk["k1_project"]["hbm_gbs"] / sg["read1_write2"], 4)
        kk["k3_output"]["hbm_frac_measured"] = round(kk["k3_output"]["hbm_gbs"] / sg["read2_write1"], 4)
        log("measured peaks: %s" % json.dumps(mp))
    if k0_ms is not None:
        result["kernels"]["k0_mask_ranges"] = {"ms": round(k0_ms, 4),
                                               "hbm_gbs": round(B * NN * es / k0_ms / 1e6, 1)}
    if cold or len(directions) > 1:
        result["per_direction_ms"] = {d: {"median": round(statistics.median(v), 4), "min": round(min(v), 4)}
                                      for d, v in per_call.items() if v}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(wl, z, mask, w, direction, args.cpu_sample)
        log("cpu baseline done")
    else:
        result["cpu_baseline"] = None
    layer.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
