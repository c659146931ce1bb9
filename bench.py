"""Benchmark of the hard (and soft) Euler characteristic curve on one MI355X.

One step = one hard ECC of an 8192^2 uint8 grid (H=256, tau_k=k) plus one
hard ECC of a 512^3 float32 Gaussian random field (H=512, linspace(min,max)),
the two workloads the headline metric (voxels/s and HBM GB/s) is quoted on.
Inputs are resident in HBM before timing; the 8192^2 input rotates over 8
distinct buffers (512 MiB in all) and the 512^3 input over 2, so repeated
steps cannot be served from the 256 MB Infinity Cache.

Also reported on the same JSON line: per-kernel durations and roofline of
each hard kernel (HIP events on the launch stream), the soft forward /
backward at 256^3 (H=256, lambda=50), and the CPU oracle timed on a bounded
sample of the same workloads (cpu_baseline).

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
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9   # non-packed 32-bit lane-ops/s: 256 CU x 4 SIMD x 16 lanes x 2.4 GHz


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


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--kernel-reps", type=int, default=40)
    ap.add_argument("--soft-reps", type=int, default=3)
    ap.add_argument("--no-soft", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def timed(torch, fn, reps):
    """Average ms per call of fn() over reps calls, HIP events on torch's current stream."""
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


def cpu_baseline(W, oracle):
    """The oracle on a bounded sample of the same two workloads, on this host."""
    g3, t3, _ = W.make_workload("c3_8192sq_u8")
    s3 = np.ascontiguousarray(g3[:1024])
    g4, t4, _ = W.make_workload("c4a_512cube_f32_grf")
    s4 = np.ascontiguousarray(g4[:32])
    t0 = time.perf_counter()
    oracle.ecc_hard(s3, t3)
    t1 = time.perf_counter()
    oracle.ecc_hard(s4, t4)
    t2 = time.perf_counter()
    vox = s3.size + s4.size
    return {
        "value": vox / (t2 - t0), "unit": "voxels/s", "cores": 1, "kind": "oracle",
        "sample": f"rows 0..1023 of the 8192^2 uint8 grid ({s3.size} px, {t1 - t0:.1f} s) + planes 0..31 "
                  f"of the 512^3 GRF ({s4.size} vox, {t2 - t1:.1f} s); numpy, single-threaded",
        "host_cpus": os.cpu_count(),
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): the ECC of "
              "one grid is a single-GPU job; the sharding design is described in DESIGN.md.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import euler_characteristic_curves_amd as E
    from euler_characteristic_curves_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    log("generating 8192^2 uint8 grid")
    g3, t3, _ = W.make_workload("c3_8192sq_u8")
    log("generating 512^3 float32 GRF")
    g4, t4, _ = W.make_workload("c4a_512cube_f32_grf")
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

    log("warmup", args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_step = timed(torch, step, args.steps)

    log("per-kernel timing")
    ms3 = timed(torch, lambda i: E.ecc_hard_2d(b3[i % 8], dt3, out=o3), args.kernel_reps)
    ms4 = timed(torch, lambda i: E.ecc_hard_3d(b4[i % 2], dt4, out=o4), args.kernel_reps)
    alg3 = n3 * 1 + 4 * 256 + 8 * 256
    alg4 = n4 * 4 + 4 * 512 + 8 * 512
    gbs3 = alg3 / (ms3 * 1e-3) / 1e9
    gbs4 = alg4 / (ms4 * 1e-3) / 1e9

    soft = None
    if not args.no_soft:
        log("soft 256^3")
        gs, ts, extra = W.make_workload("c5_256cube_soft")
        dgs, dts = torch.from_numpy(gs).to(dev), torch.from_numpy(ts).to(dev)
        dgo = torch.from_numpy(extra["grad_out"]).to(dev)
        lam = extra["lam"]
        E.ecc_soft_fwd(dgs, dts, lam)
        E.ecc_soft_bwd_tau(dgs, dts, lam, dgo)
        msf = timed(torch, lambda i: E.ecc_soft_fwd(dgs, dts, lam), args.soft_reps)
        msb = timed(torch, lambda i: E.ecc_soft_bwd_tau(dgs, dts, lam, dgo), args.soft_reps)
        pairs = n_cells(gs.shape) * ts.size
        soft = {
            "workload": "soft ECC 256^3 float32 uniform, H=256, lambda=50",
            "fwd_ms": msf, "bwd_ms": msb,
            "cell_threshold_pairs": pairs,
            "fwd_pairs_per_s": pairs / (msf * 1e-3), "bwd_pairs_per_s": pairs / (msb * 1e-3),
        }

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        import oracle
        cpu = cpu_baseline(W, oracle)

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
            "frac": gbs4 / HBM_PEAK_GBS, "traffic": None,
            "kernel": "hard3d_kernel (512^3 float32, H=512)", "ms_per_launch": ms4,
            "algorithmic_bytes_per_launch": alg4,
        },
        "kernels": {
            "hard_8192sq_u8": {"ms": ms3, "voxels_per_s": n3 / (ms3 * 1e-3), "GB_s": gbs3,
                               "frac_hbm_peak": gbs3 / HBM_PEAK_GBS, "algorithmic_bytes": alg3},
            "hard_512cube_f32": {"ms": ms4, "voxels_per_s": n4 / (ms4 * 1e-3), "GB_s": gbs4,
                                 "frac_hbm_peak": gbs4 / HBM_PEAK_GBS, "algorithmic_bytes": alg4},
        },
        "soft": soft,
        "cpu_baseline": cpu,
        "context": {"rtx_a6000_ms": {"8192sq": 1.6, "512cube": 5.61, "1024sq": 0.032, "1024cube": 48.47}},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
