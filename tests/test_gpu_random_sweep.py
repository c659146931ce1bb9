"""GPU parity over seeded random sweeps of hard- and soft-ECC cases.

Each case draws a 2D or 3D shape (up to 1.5 M voxels, any row length, so
aligned and unaligned rows, full and partial column chunks), a value kind
(uint8, uniform float32, float32 with many ties, a wide normal field), a
threshold count H and a threshold kind (evenly spaced over the data, drawn
from the data's own values with repeats, unsorted and outside the data range,
or the data's quantiles), and compares the HIP result with the oracle bit for
bit.  The soft sweep draws small grids, lambda and thresholds the same way and
checks the forward, dL/dtau and dL/dgrid against the float64 oracle within the
soft tolerance.  Every case names itself on stdout before its GPU step.
"""

import numpy as np
import pytest

import oracle
from euler_characteristic_curves_amd import workloads as W
from tests.gpu_util import banner, need_gpu, soft_close

pytestmark = pytest.mark.gpu

CASES_PER_SEED = 12
SEEDS = list(range(10))


@pytest.fixture(scope="module")
def E():
    need_gpu()
    import euler_characteristic_curves_amd as E
    return E


def _draw(rng):
    nd = int(rng.integers(2, 4))
    while True:
        dims = ([int(rng.integers(1, 48))] if nd == 3 else []) + [int(rng.integers(1, 400)),
                                                                   int(rng.integers(1, 1100))]
        if np.prod(dims) <= 1_500_000:
            break
    shape = tuple(dims)
    kind = str(rng.choice(["u8", "f32", "f32ties", "f32wide"]))
    if kind == "u8":
        g = rng.integers(0, 256, size=shape, dtype=np.uint8)
    elif kind == "f32":
        g = rng.random(shape, dtype=np.float32)
    elif kind == "f32ties":
        g = rng.integers(0, 7, size=shape).astype(np.float32)
    else:
        g = (rng.standard_normal(shape) * 3).astype(np.float32)
    H = int(rng.choice([1, 2, 3, 17, 97, 255, 256, 257, 511, 512, 1024, 2048]))
    tk = str(rng.choice(["linspace", "dups", "unsorted", "quantile"]))
    lo, hi = float(g.min()), float(g.max())
    if tk == "linspace":
        tau = W.tau_linspace(lo, hi, H)
    elif tk == "dups":
        tau = np.sort(rng.choice(np.unique(g.astype(np.float32)), size=H)).astype(np.float32)
    elif tk == "unsorted":
        tau = rng.uniform(lo - 1, hi + 1, size=H).astype(np.float32)
    else:
        tau = np.quantile(g.astype(np.float64), np.linspace(0, 1, H)).astype(np.float32)
    return g, tau, f"{shape} {kind} H={H} {tk}"


@pytest.mark.parametrize("seed", SEEDS)
def test_hard_random_sweep(E, seed):
    import torch
    rng = np.random.default_rng(1000 + seed)
    for i in range(CASES_PER_SEED):
        g, tau, name = _draw(rng)
        want = oracle.ecc_hard(g, tau)
        banner("hard sweep", seed, i, name)
        got = E.ecc_hard(torch.from_numpy(g).cuda(), torch.from_numpy(tau).cuda()).cpu().numpy()
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"{name}: {bad.size} mismatches, first k={bad[:5]}"


SOFT_CASES_PER_SEED = 4
SOFT_SEEDS = list(range(5))


@pytest.mark.parametrize("seed", SOFT_SEEDS)
def test_soft_random_sweep(E, seed):
    """Soft forward, dL/dtau and dL/dgrid on seeded random small grids, within
    1e-4 relative where |value| >= 10, else 1e-3 absolute, of the float64
    oracle; lambda from 0.5 to 2000 and thresholds evenly spaced (sometimes
    beyond the data), unsorted or repeated."""
    import torch
    rng = np.random.default_rng(2000 + seed)
    for i in range(SOFT_CASES_PER_SEED):
        nd = int(rng.integers(2, 4))
        while True:
            dims = ([int(rng.integers(1, 24))] if nd == 3 else []) + [int(rng.integers(1, 80)),
                                                                       int(rng.integers(1, 300))]
            if np.prod(dims) <= 20_000:
                break
        shape = tuple(dims)
        g = rng.random(shape, dtype=np.float32)
        if rng.random() < 0.3:
            g = (np.round(g * 8) / 8).astype(np.float32)  # many ties
        H = int(rng.choice([1, 5, 64, 256, 300]))
        lam = float(rng.choice([0.5, 5.0, 50.0, 400.0, 2000.0]))
        tk = str(rng.choice(["linspace", "wide", "unsorted", "dups"]))
        if tk == "linspace":
            tau = W.tau_linspace(-0.05, 1.05, H)
        elif tk == "wide":
            tau = W.tau_linspace(-3.0, 4.0, H)
        elif tk == "unsorted":
            tau = rng.uniform(-0.2, 1.2, size=H).astype(np.float32)
        else:
            tau = np.sort(rng.choice(np.unique(g), size=H)).astype(np.float32)
        gout = rng.standard_normal(H).astype(np.float32)
        name = f"{shape} H={H} lam={lam:g} {tk}"
        dg, dt, dgo = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (g, tau, gout))
        banner("soft sweep fwd", seed, i, name)
        f = E.ecc_soft_fwd(dg, dt, lam).cpu().numpy()
        bad, worst = soft_close(f, oracle.ecc_soft(g, tau, lam))
        assert bad.size == 0, (name, "fwd", bad[:5], worst)
        banner("soft sweep bwd tau", seed, i, name)
        b = E.ecc_soft_bwd_tau(dg, dt, lam, dgo).cpu().numpy()
        bad, worst = soft_close(b, oracle.ecc_soft_bwd_tau(g, tau, lam, gout))
        assert bad.size == 0, (name, "bwd tau", bad[:5], worst)
        banner("soft sweep bwd grid", seed, i, name)
        gg = E.ecc_soft_bwd_grid(dg, dt, lam, dgo).cpu().numpy()
        bad, worst = soft_close(gg.ravel(), oracle.ecc_soft_bwd_grid(g, tau, lam, gout).ravel())
        assert bad.size == 0, (name, "bwd grid", bad[:5], worst)
