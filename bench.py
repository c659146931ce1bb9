"""Benchmark of the hard (and soft) Euler characteristic curve on one MI355X.

One step = one hard ECC of an 8192^2 uint8 grid (H=256, tau_k=k) plus one
hard ECC of a 512^3 float32 Gaussian random field (H=512, linspace(min,max)),
the two workloads the headline metric (voxels/s and HBM GB/s) is quoted on.
Inputs are resident in HBM before timing; the 8192^2 input rotates over 8
distinct buffers (512 MiB in all) and the 512^3 input over 2, so repeated
steps cannot be served from the 256 MB Infinity Cache.

Also reported on the same JSON line: per-kernel durations (mean of
back-to-back launches, and min / median of individually timed launches, HIP
events on the launch stream) and the roofline of each hard kernel; the other
grid sizes (128^2, 1024^2, 1024^3) as context, the first two also as batches
of 1024 and 64 grids in one call, and curves of a 128^3 grid along 64 / 16
directions (hard / soft with all gradients); the soft forward and its
backward with respect to the thresholds and to the grid at 256^3 (H=256,
lambda=50) with their VALU-issue fraction; and the CPU oracle
timed on a bounded sample of the same workloads (cpu_baseline), on one core
and on all cores, before the GPU is touched.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD public spec
VALU_WAVE_INSTR_PEAK = 256 * 2.4e9    # wave64 VALU instructions/s: one per CU per clock (4 SIMD x 16 lanes)


def n_cells(shape):
    """Number of cells of the V-construction complex of a box (all dimensions)."""
    import itertools
    total = 0
    for ext in itertools.product((0, 1), repeat=len(shape)):
        n = 1
        for s, e in zip(shape, ext):
            n *= s - e
        total += n
    return total


KERNEL_SOURCES = ("euler_characteristic_curves_amd/csrc/ecc_hard.hip",
                  "euler_characteristic_curves_amd/csrc/ecc_device.hpp",
                  "euler_characteristic_curves_amd/csrc/ecc_internal.hpp")
TRAFFIC_PROFILE = "profiles/hard3d_512cube_f32_traffic.md"
TRAFFIC_PROFILE_U8 = "profiles/hard2d_8192sq_u8_traffic.md"
SOFT_SOURCES = ("euler_characteristic_curves_amd/csrc/ecc_soft.hip",
                "euler_characteristic_curves_amd/csrc/ecc_soft_grad.hip",
                "euler_characteristic_curves_amd/csrc/ecc_star.hpp",
                "euler_characteristic_curves_amd/csrc/ecc_device.hpp",
                "euler_characteristic_curves_amd/csrc/ecc_internal.hpp")
SQ_PROFILE = "profiles/ecc_kernels_bench_sq_counters.md"


def source_hash(files):
    """sha256 over the given kernel sources."""
    import hashlib
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_source_hash():
    """sha256 over the sources the hard kernels are built from."""
    return source_hash(KERNEL_SOURCES)


def profile_fields(rel):
    """`name: value` lines of a committed profile summary (backticks stripped)."""
    path = os.path.join(ROOT, rel)
    fields = {}
    if not os.path.exists(path):
        return fields
    with open(path) as f:
        for line in f:
            t = line.strip()
            if t and ":" in t and not t.startswith(("#", "|", "`")) and " " not in t.split(":", 1)[0]:
                k, v = t.split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    return fields


def recorded_traffic(profile=TRAFFIC_PROFILE):
    """HBM bytes per launch of a hard kernel from its committed rocprofv3 --pmc profile.

    Returns None unless the profile was taken on the current kernel sources
    (its `kernel_source_sha256:` line matches), so a stale figure is never
    reported.
    """
    fields = profile_fields(profile)
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def recorded_soft_valu(kind="issue"):
    """(forward, tau-backward, grid-backward) VALU work per soft launch at
    256^3, H=256, from the committed rocprofv3 SQ profile.

    kind="issue": SQ_ACTIVE_INST_VALU, the VALU issue slots the waves occupy
    (a transcendental takes two); kind="instr": SQ_INSTS_VALU, instructions.
    Both are fixed by the kernels and their input, and are used only while the
    soft sources hash to the value recorded in the profile.
    """
    fields = profile_fields(SQ_PROFILE)
    if fields.get("soft_source_sha256") != source_hash(SOFT_SOURCES):
        return None, None, None
    suffix = {"issue": "valu_issue_slots", "instr": "valu_wave_instr", "trans": "valu_trans_instr"}[kind]
    out = []
    for op in ("fwd", "bwd", "grad"):
        try:
            out.append(float(fields[f"soft_{op}_{suffix}"]))
        except (KeyError, ValueError):
            out.append(None)
    return tuple(out)


def traffic_run():
    """Workload for the two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE).

    Runs a plain 512 MiB device-to-device copy (the calibration kernel of
    known size) three times, then the hard 3D kernel on the 512^3 float32
    field three times, then the hard 2D kernel on three different 8192^2
    uint8 grids.
    """
    import torch

    import euler_characteristic_curves_amd as E
    from euler_characteristic_curves_amd import workloads as W
    dev = torch.device("cuda:0")
    g4, t4, _ = W.make_workload("c4a_512cube_f32_grf")
    d4 = torch.from_numpy(g4).to(dev)
    dst = torch.empty_like(d4)
    dt4 = torch.from_numpy(t4).to(dev)
    for _ in range(3):
        dst.copy_(d4)
    torch.cuda.synchronize()
    for _ in range(3):
        E.ecc_hard_3d(d4, dt4)
    torch.cuda.synchronize()
    g3, t3, _ = W.make_workload("c3_8192sq_u8")
    d3 = [torch.from_numpy(np.roll(g3, k, axis=0)).to(dev) for k in range(3)]
    dt3 = torch.from_numpy(t3).to(dev)
    torch.cuda.synchronize()
    for k in range(3):
        E.ecc_hard_2d(d3[k], dt3)
    torch.cuda.synchronize()
    print("traffic run done: copy bytes", d4.numel() * 4, flush=True)


def soft_sweep_terms(g):
    """Number of (value, weight) terms the soft sweep evaluates for grid g.

    Mirrors how the sweep builds its terms (measurement only; the result does
    not enter any curve): per voxel, the four row sequences of the telescoped
    regrouping (the row, the max over y, over z, and over y and z), each with
    weight inc(x) - inc(x-1), signed +, -, -, +; equal values within a voxel
    are merged, and terms of weight 0 or of cells outside the grid dropped.
    The sweep evaluates terms x H sigmoids.
    """
    inf = np.float32(np.inf)
    g = g.reshape((1,) * (3 - g.ndim) + g.shape).astype(np.float32, copy=False)
    nz, ny, nx = g.shape
    col = np.full((ny, 1), inf, np.float32)
    row = np.full((1, nx), inf, np.float32)
    total = 0
    for z in range(nz):
        a = g[z]
        b = g[z + 1] if z + 1 < nz else np.full_like(a, inf)
        ay, by = np.vstack([a[1:], row]), np.vstack([b[1:], row])
        v = [a, np.maximum(a, ay), np.maximum(a, b), np.maximum(np.maximum(a, ay), np.maximum(b, by))]
        w = []
        for q, c in enumerate(v):
            left, right = np.hstack([col, c[:, :-1]]), np.hstack([c[:, 1:], col])
            wq = (right > c).astype(np.int32) - (c > left).astype(np.int32)
            w.append(-wq if q in (1, 2) else wq)
        m = v[3] == v[2]
        w[2], w[3] = np.where(m, w[2] + w[3], w[2]), np.where(m, 0, w[3])
        m = (v[3] == v[1]) & (w[3] != 0)
        w[1], w[3] = np.where(m, w[1] + w[3], w[1]), np.where(m, 0, w[3])
        m = v[2] == v[1]
        w[1], w[2] = np.where(m, w[1] + w[2], w[1]), np.where(m, 0, w[2])
        m = v[1] == v[0]
        w[0], w[1] = np.where(m, w[0] + w[1], w[0]), np.where(m, 0, w[1])
        m = v[2] == v[0]
        w[0], w[2] = np.where(m, w[0] + w[2], w[0]), np.where(m, 0, w[2])
        total += sum(int(np.count_nonzero((wq != 0) & (vq < inf))) for vq, wq in zip(v, w))
    return total


def sigmoid_ceiling(torch, cus):
    """Measured pairs/s of the soft sweep's per-pair arithmetic with every
    operand in registers (libecc_sigmoid_rate.so): (forward, backward)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "euler_characteristic_curves_amd", "libecc_sigmoid_rate.so"))
    lib.ecc_sigmoid_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.ecc_sigmoid_rate.restype = ctypes.c_int
    blocks, iters = 8 * cus, 2048
    out = torch.empty(blocks * 256, dtype=torch.float64, device="cuda:0")
    s = torch.cuda.current_stream()
    rates = []
    for bwd in (0, 1):
        def run(i):
            st = lib.ecc_sigmoid_rate(bwd, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                                      ctypes.c_void_p(s.cuda_stream))
            if st != 0:
                raise RuntimeError(f"ecc_sigmoid_rate failed with HIP error {st}")
        run(0)
        ms = min(timed(torch, run, 3) for _ in range(3))
        rates.append(blocks * 256 * iters * 8 / (ms * 1e-3))
    return tuple(rates)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--kernel-reps", type=int, default=50)
    ap.add_argument("--soft-reps", type=int, default=5)
    ap.add_argument("--no-soft", action="store_true")
    ap.add_argument("--no-context", action="store_true", help="skip the 128^2 / 1024^2 / 1024^3 timings")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-run", action="store_true",
                    help="only run the workload profiled for HBM traffic (under rocprofv3 --pmc)")
    return ap.parse_args()


def spin_up(torch, fn, seconds):
    """Run fn(i) untimed until `seconds` of wall time have passed.

    The GPU raises its clocks only after some milliseconds of sustained work:
    back-to-back 1024^3 launches measured 1.1-1.5 ms for the first ten after an
    idle gap and 0.99 ms from then on, and launches 50 ms apart 1.04-1.14 ms.
    Timing starts once the clocks have left the idle state.
    """
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def timed(torch, fn, reps):
    """Mean ms per call of fn(i) over reps back-to-back calls (HIP events on the current stream)."""
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for i in range(reps):
        fn(i)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def timed_each(torch, fn, reps):
    """(min, median) ms of reps individually bracketed calls of fn(i)."""
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record(s)
        fn(i)
        b.record(s)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[0], t[len(t) // 2]


# ------------------------------------------------------------ CPU baseline
_CPU = {}


def _cpu_work(i):
    """One worker's share of the all-core oracle run: a 1024-row band of the
    8192^2 grid and a 32-plane slab of the 512^3 field (hard ECC of each)."""
    import oracle
    g3, t3, g4, t4 = _CPU["g3"], _CPU["t3"], _CPU["g4"], _CPU["t4"]
    r = (i % 8) * 1024
    z = (i % 16) * 32
    oracle.ecc_hard(np.ascontiguousarray(g3[r:r + 1024]), t3)
    oracle.ecc_hard(np.ascontiguousarray(g4[z:z + 32]), t4)
    return 1024 * g3.shape[1] + 32 * g4.shape[1] * g4.shape[2]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W, g3, t3, g4, t4):
    """The oracle on a bounded sample of the two bench workloads, on this host.

    Runs before anything touches the GPU (the all-core leg forks workers).
    One core: rows 0..4095 of the 8192^2 grid and planes 0..127 of the 512^3
    field.  All cores: one worker per available core (at most 16), each on a
    1024-row band and a 32-plane slab (histograms of disjoint owners add, so
    this is the oracle's natural parallel form); throughput = voxels / wall.
    """
    import multiprocessing as mp

    import oracle
    s3 = np.ascontiguousarray(g3[:4096])
    s4 = np.ascontiguousarray(g4[:128])
    t0 = time.perf_counter()
    oracle.ecc_hard(s3, t3)
    t1 = time.perf_counter()
    oracle.ecc_hard(s4, t4)
    t2 = time.perf_counter()
    one = (s3.size + s4.size) / (t2 - t0)

    try:
        ncores = len(os.sched_getaffinity(0))
    except AttributeError:
        ncores = os.cpu_count() or 1
    ncores = max(1, min(ncores, 16))
    _CPU.update(g3=g3, t3=t3, g4=g4, t4=t4)
    ctx = mp.get_context("fork")
    with ctx.Pool(ncores) as pool:
        t3a = time.perf_counter()
        vox = sum(pool.map(_cpu_work, range(ncores)))
        t4a = time.perf_counter()
    _CPU.clear()
    return {
        "value": one, "unit": "voxels/s", "cores": 1, "kind": "oracle",
        "sample": f"rows 0..4095 of the 8192^2 uint8 grid ({s3.size} px, {t1 - t0:.1f} s) + planes 0..127 "
                  f"of the 512^3 GRF ({s4.size} vox, {t2 - t1:.1f} s); numpy, single-threaded",
        "all_cores": {"value": vox / (t4a - t3a), "unit": "voxels/s", "cores": ncores,
                      "sample": f"{ncores} workers, each a 1024-row band of the 8192^2 grid + a 32-plane slab "
                                f"of the 512^3 GRF ({vox} voxels in {t4a - t3a:.1f} s wall)"},
        "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
    }


def directional_context(torch, E, W, dev, reps):
    """Curves of a 128^3 float32 uniform grid along many directions: heights
    f_d = X + <u_d, p> (HBM-bound elementwise kernel), then the hard curves of
    all D height grids in one batched call (64 directions, H=256), and the soft
    curves with every gradient (16 directions, H=128, lambda=20)."""
    rng = np.random.default_rng(77)
    X = W.uniform_f32((128, 128, 128), 78)
    dX = torch.from_numpy(X).to(dev)
    out = {}
    for D, soft in ((64, False), (16, True)):
        U = rng.normal(size=(D, 3))
        U = (U / np.linalg.norm(U, axis=1, keepdims=True)).astype(np.float32)
        dU = torch.from_numpy(U).to(dev)
        dA = torch.ones(D, dtype=torch.float32, device=dev)
        f = E.ecc_height(dX, dU, dA)
        lo, hi = float(f.min().item()), float(f.max().item())
        ms_h = timed(torch, lambda i: E.ecc_height(dX, dU, dA, out=f), reps)
        bytes_h = X.size * 4 * (1 + D)
        rec = {"directions": D, "height_ms": ms_h, "height_GB_s": bytes_h / (ms_h * 1e-3) / 1e9,
               "height_frac_hbm_peak": bytes_h / (ms_h * 1e-3) / 1e9 / HBM_PEAK_GBS}
        if not soft:
            tau = torch.from_numpy(W.tau_linspace(lo, hi, 256)).to(dev)
            o = torch.empty((D, 256), dtype=torch.int64, device=dev)
            ms_c = timed(torch, lambda i: E.ecc_hard_batched(f, tau, out=o), reps)
            rec.update({"H": 256, "hard_curves_ms": ms_c, "total_ms": ms_h + ms_c,
                        "voxel_directions_per_s": X.size * D / ((ms_h + ms_c) * 1e-3)})
            out["hard"] = rec
        else:
            tau = torch.from_numpy(W.tau_linspace(lo, hi, 128)).to(dev)
            w = torch.from_numpy(rng.standard_normal((D, 128)).astype(np.float32)).to(dev)
            xg = dX.clone().requires_grad_(True)
            ug = dU.clone().requires_grad_(True)
            ag = dA.clone().requires_grad_(True)
            tg = tau.clone().requires_grad_(True)

            def step(i):
                S = E.soft_ecc_directional(xg, ug, ag, tg, 20.0)
                (S * w).sum().backward()

            for i in range(3):  # the first backward passes load torch's gradient-accumulation kernels
                step(i)
            ms_fb = timed(torch, step, max(3, reps // 5))
            ms_fw = timed(torch, lambda i: E.soft_ecc_directional(dX, dU, dA, tau, 20.0), max(3, reps // 5))
            rec.update({"H": 128, "lambda": 20.0, "soft_forward_ms": ms_fw, "soft_forward_backward_ms": ms_fb})
            out["soft"] = rec
        del f
    del dX
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): the ECC of "
              "one grid is a single-GPU job, and sharding a grid over several GPUs is not built.",
              file=sys.stderr)
        sys.exit(2)

    if args.traffic_run:
        traffic_run()
        return

    from euler_characteristic_curves_amd import workloads as W

    log("generating 8192^2 uint8 grid")
    g3, t3, _ = W.make_workload("c3_8192sq_u8")
    log("generating 512^3 float32 GRF")
    g4, t4, _ = W.make_workload("c4a_512cube_f32_grf")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample, before the GPU is touched)")
        cpu = cpu_baseline(W, g3, t3, g4, t4)

    import torch

    import euler_characteristic_curves_amd as E

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    n3, n4 = g3.size, g4.size
    b3 = [torch.from_numpy(g3).to(dev) for _ in range(8)]
    d4 = torch.from_numpy(g4).to(dev)
    b4 = [d4, d4.clone()]
    dt3 = torch.from_numpy(t3).to(dev)
    dt4 = torch.from_numpy(t4).to(dev)
    o3 = torch.empty(256, dtype=torch.int64, device=dev)
    o4 = torch.empty(512, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()

    def step(i):
        E.ecc_hard_2d(b3[i % 8], dt3, out=o3)
        E.ecc_hard_3d(b4[i % 2], dt4, out=o4)

    log("clock spin-up (untimed)")
    spin_up(torch, step, 0.3)
    log("warmup", args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_step = timed(torch, step, args.steps)

    log("per-kernel timing")
    f3 = lambda i: E.ecc_hard_2d(b3[i % 8], dt3, out=o3)
    f4 = lambda i: E.ecc_hard_3d(b4[i % 2], dt4, out=o4)
    ms3, ms4 = timed(torch, f3, args.kernel_reps), timed(torch, f4, args.kernel_reps)
    mm3, mm4 = timed_each(torch, f3, args.kernel_reps), timed_each(torch, f4, args.kernel_reps)
    alg3 = n3 * 1 + 4 * 256 + 8 * 256
    alg4 = n4 * 4 + 4 * 512 + 8 * 512
    gbs3 = alg3 / (ms3 * 1e-3) / 1e9
    gbs4 = alg4 / (ms4 * 1e-3) / 1e9
    del b3
    torch.cuda.empty_cache()

    context = None
    if not args.no_context:
        context = {"rtx_a6000_ms_from_the_pages": {"1024sq": 0.032, "8192sq": 1.6, "512cube": 5.61,
                                                   "1024cube": 48.47}}
        for name in ("c1_128sq_f32", "c2_1024sq_f32_grf", "c4b_1024cube_f32"):
            log("context", name)
            g, tau, _ = W.make_workload(name)
            dg, dtau = torch.from_numpy(g).to(dev), torch.from_numpy(tau).to(dev)
            del g
            o = torch.empty(dtau.numel(), dtype=torch.int64, device=dev)
            fn = lambda i: E.ecc_hard(dg, dtau, out=o)
            spin_up(torch, fn, 0.1)
            reps = 10 if dg.numel() > 1e8 else args.kernel_reps
            ms = timed(torch, fn, reps)
            mn, md = timed_each(torch, fn, reps)
            context[name] = {"shape": list(dg.shape), "H": int(dtau.numel()), "ms": ms, "min_ms": mn,
                             "median_ms": md, "voxels_per_s": dg.numel() / (ms * 1e-3),
                             "GB_s": (dg.numel() * dg.element_size() + 12 * dtau.numel()) / (ms * 1e-3) / 1e9}
            if name != "c4b_1024cube_f32":
                # the same grid size as a batch: B distinct grids (rolled copies of
                # this one), one call, one curve per grid
                B = 1024 if name == "c1_128sq_f32" else 64
                log("context batched", name, B)
                gb = torch.stack([torch.roll(dg, shifts=(7 * b, 13 * b), dims=(0, 1)) for b in range(B)])
                ob = torch.empty((B, dtau.numel()), dtype=torch.int64, device=dev)
                fb = lambda i: E.ecc_hard_batched(gb, dtau, out=ob)
                spin_up(torch, fb, 0.1)
                msb = timed(torch, fb, args.kernel_reps)
                context[name]["batched"] = {
                    "batch": B, "ms": msb, "us_per_grid": msb * 1e3 / B,
                    "voxels_per_s": gb.numel() / (msb * 1e-3),
                    "GB_s": (gb.numel() * gb.element_size() + 12 * dtau.numel()) / (msb * 1e-3) / 1e9,
                    "speedup_per_grid_vs_single_calls": ms * B / msb}
                del gb, ob
            del dg, dtau, o
            torch.cuda.empty_cache()
        context["directional_128cube"] = directional_context(torch, E, W, dev, args.kernel_reps)

    soft = None
    if not args.no_soft:
        log("soft 256^3")
        gs, ts, extra = W.make_workload("c5_256cube_soft")
        dgs, dts = torch.from_numpy(gs).to(dev), torch.from_numpy(ts).to(dev)
        dgo = torch.from_numpy(extra["grad_out"]).to(dev)
        lam = extra["lam"]
        dgg = torch.empty_like(dgs)
        E.ecc_soft_fwd(dgs, dts, lam)
        E.ecc_soft_bwd_tau(dgs, dts, lam, dgo)
        E.ecc_soft_bwd_grid(dgs, dts, lam, dgo, dgg)
        spin_up(torch, lambda i: E.ecc_soft_fwd(dgs, dts, lam), 0.1)
        msf = timed(torch, lambda i: E.ecc_soft_fwd(dgs, dts, lam), args.soft_reps)
        msb = timed(torch, lambda i: E.ecc_soft_bwd_tau(dgs, dts, lam, dgo), args.soft_reps)
        msg = timed(torch, lambda i: E.ecc_soft_bwd_grid(dgs, dts, lam, dgo, dgg), args.soft_reps)
        torch.cuda.synchronize()
        grad_nonzero = int(torch.count_nonzero(dgg).item())
        pairs = n_cells(gs.shape) * ts.size
        nf, nb, ng = recorded_soft_valu("instr")
        vf, vb, vg = recorded_soft_valu("issue")
        tf, tb, tg = recorded_soft_valu("trans")

        def minus(a, b):
            return None if a is None or b is None else a - b

        def frac(v, ms):
            return None if v is None else v / (ms * 1e-3) / VALU_WAVE_INSTR_PEAK

        sig = soft_sweep_terms(gs) * ts.size
        cf_rate, cb_rate = sigmoid_ceiling(torch, torch.cuda.get_device_properties(0).multi_processor_count)
        soft = {
            "workload": "soft ECC 256^3 float32 uniform, H=256, lambda=50",
            "fwd_ms": msf, "bwd_ms": msb, "fwd_plus_bwd_ms": msf + msb,
            "cell_threshold_pairs": pairs,
            "fwd_pairs_per_s": pairs / (msf * 1e-3), "bwd_pairs_per_s": pairs / (msb * 1e-3),
            # sigmoids the sweep actually evaluates (merged terms x H), their
            # rate, and the rate of the same per-pair arithmetic measured with
            # every operand in registers on this GPU
            "sigmoids_per_pass": sig,
            "fwd_sigmoids_per_s": sig / (msf * 1e-3), "bwd_sigmoids_per_s": sig / (msb * 1e-3),
            "sigmoid_ceiling_per_s": {"fwd": cf_rate, "bwd": cb_rate},
            "sigmoid_ceiling_frac": {"fwd": sig / (msf * 1e-3) / cf_rate, "bwd": sig / (msb * 1e-3) / cb_rate},
            "bwd_grid_ms": msg,
            "bwd_grid_voxels_per_s": gs.size / (msg * 1e-3),
            "bwd_grid_nonzero_voxels": grad_nonzero,
            "bwd_grid_voxel_threshold_pairs_per_s": grad_nonzero * ts.size / (msg * 1e-3),
            # fractions of the VALU issue rate by count of the instructions
            # other than transcendentals (v_exp / v_rcp run beside them: with
            # them counted the backward passes 100 %); all VALU instructions
            # and the issue slots (a transcendental occupies two) beside them
            "roofline": {"bound": "valu", "unit": "wave64 VALU instr/s, transcendentals excluded",
                         "peak": VALU_WAVE_INSTR_PEAK,
                         "fwd_frac": frac(minus(nf, tf), msf), "bwd_frac": frac(minus(nb, tb), msb),
                         "bwd_grid_frac": frac(minus(ng, tg), msg),
                         "valu_instr_per_launch": {"fwd": nf, "bwd": nb, "bwd_grid": ng},
                         "trans_instr_per_launch": {"fwd": tf, "bwd": tb, "bwd_grid": tg},
                         "all_valu_frac": {"fwd": frac(nf, msf), "bwd": frac(nb, msb), "bwd_grid": frac(ng, msg)},
                         "valu_issue_slots_per_launch": {"fwd": vf, "bwd": vb, "bwd_grid": vg},
                         "issue_slot_frac": {"fwd": frac(vf, msf), "bwd": frac(vb, msb), "bwd_grid": frac(vg, msg)}},
        }

    vox_step = n3 + n4
    line = {
        "metric": "voxels/s & HBM GB/s (% of peak) for hard ECC at 8192^2 2D and 512^3 3D",
        "value": vox_step / (ms_step * 1e-3),
        "unit": "voxels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int64",
        "data": "synthetic",
        "config": {
            "workload": "hard ECC: 8192x8192 uint8 iid uniform (H=256, tau_k=k) + 512^3 float32 Gaussian "
                        "random field sigma=3 (H=512, linspace(min,max)), one of each per step",
            "voxels_per_step": vox_step,
            "rotating_buffers": {"8192sq_u8": 8, "512cube_f32": 2},
        },
        "roofline": {
            "bound": "hbm", "achieved": gbs4, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs4 / HBM_PEAK_GBS, "traffic": recorded_traffic(),
            "kernel": "hard3d_kernel (512^3 float32, H=512)", "ms_per_launch": ms4,
            "algorithmic_bytes_per_launch": alg4,
        },
        "kernels": {
            "hard_8192sq_u8": {"ms": ms3, "min_ms": mm3[0], "median_ms": mm3[1],
                               "traffic": recorded_traffic(TRAFFIC_PROFILE_U8),
                               "voxels_per_s": n3 / (ms3 * 1e-3), "GB_s": gbs3,
                               "frac_hbm_peak": gbs3 / HBM_PEAK_GBS, "algorithmic_bytes": alg3},
            "hard_512cube_f32": {"ms": ms4, "min_ms": mm4[0], "median_ms": mm4[1],
                                 "voxels_per_s": n4 / (ms4 * 1e-3), "GB_s": gbs4,
                                 "frac_hbm_peak": gbs4 / HBM_PEAK_GBS, "algorithmic_bytes": alg4},
        },
        "soft": soft,
        "cpu_baseline": cpu,
        "context": context,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
