"""Running the oracle on z-slabs of large 3D grids, in worker processes.

Test infrastructure: every number comes from ``oracle/``; this module only
cuts grids into slabs and adds the slab results up.

* Curves (hard, soft, dL/dtau) are sums over cells.  The cells of
  grid[z0:z1+1] are those anchored in planes z0..z1-1 plus those lying wholly
  in plane z1 (two disjoint sets), so a slab's own part is
  curve(grid[z0:z1+1]) - curve(grid[z1:z1+1]): exact for the integer hard
  curve, up to float64 rounding for the soft sums.
* The grid gradient at a voxel of plane z depends only on the cells that hold
  the voxel, which lie in planes z-1..z+1, so planes z0..z1-1 of the gradient
  of grid[z0-1:z1+1] equal those of the whole grid's gradient (slicing along
  z keeps the index order of every cell's corners, so ties go the same way).
"""

import multiprocessing as mp
import os

import numpy as np

import oracle


def slab_bounds(nz, slab):
    return [(z0, min(z0 + slab, nz)) for z0 in range(0, nz, slab)]


def curve_part(fn, grid, z0, z1):
    """fn's sum over the cells anchored in planes z0..z1-1 of a 3D grid."""
    nz = grid.shape[0]
    if z1 >= nz:
        return fn(grid[z0:nz])
    return fn(grid[z0:z1 + 1]) - fn(grid[z1:z1 + 1])


def grad_planes(grid, tau, lam, gout, z0, z1):
    """Planes z0..z1-1 of oracle.ecc_soft_bwd_grid(grid, ...)."""
    lo, hi = max(z0 - 1, 0), min(z1 + 1, grid.shape[0])
    r = oracle.ecc_soft_bwd_grid(grid[lo:hi], tau, lam, gout)
    return r[z0 - lo:z1 - lo]


def _curve_fn(kind, tau, lam):
    if kind == "hard":
        return lambda s: oracle.ecc_hard(s, tau)
    if kind == "soft":
        return lambda s: oracle.ecc_soft(s, tau, lam)
    ones = np.ones(tau.size, np.float32)
    return lambda s: oracle.ecc_soft_bwd_tau(s, tau, lam, ones)


_G = {}


def _fork_job(args):
    kind, z0, z1 = args
    return curve_part(_curve_fn(kind, _G["tau"], _G["lam"]), _G["grid"], z0, z1)


def curve_combined(kind, grid, tau, lam=None, slab=32, workers=1):
    """The whole curve ("hard", "soft", or "bwd" = dL/dtau for g = 1) as a sum
    of slab parts, in a fork pool of ``workers`` (only in processes that have
    not touched a GPU)."""
    jobs = [(kind, z0, z1) for z0, z1 in slab_bounds(grid.shape[0], slab)]
    _G.update(grid=grid, tau=tau, lam=lam)
    try:
        if workers > 1:
            with mp.get_context("fork").Pool(workers) as pool:
                parts = pool.map(_fork_job, jobs, chunksize=1)
        else:
            parts = [_fork_job(j) for j in jobs]
    finally:
        _G.clear()
    total = parts[0].copy()
    for p in parts[1:]:
        total += p
    return total


def _workload_grad_job(args):
    name, shape, z0, z1 = args
    from euler_characteristic_curves_amd import workloads as W
    g, tau, extra = W.make_workload(name, shape=shape)
    return z0, grad_planes(g, tau, extra["lam"], extra["grad_out"], z0, z1)


def workload_grad(name, shape=None, slab=16, workers=None):
    """The oracle's whole grid gradient of a named soft workload, float64.

    Workers are fresh interpreters (spawn), so this may run in a process that
    uses the GPU; each regenerates the seeded input and works on its slab.
    """
    from euler_characteristic_curves_amd import workloads as W
    shape = tuple(shape) if shape is not None else W.WORKLOADS[name]["shape"]
    if workers is None:
        try:
            workers = len(os.sched_getaffinity(0))
        except AttributeError:
            workers = os.cpu_count() or 1
    workers = max(1, min(workers, 16))
    jobs = [(name, shape, z0, z1) for z0, z1 in slab_bounds(shape[0], slab)]
    out = np.empty(shape, np.float64)
    with mp.get_context("spawn").Pool(min(workers, len(jobs))) as pool:
        for z0, planes in pool.imap_unordered(_workload_grad_job, jobs):
            out[z0:z0 + planes.shape[0]] = planes
    return out
