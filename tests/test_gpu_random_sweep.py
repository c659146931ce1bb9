"""GPU parity over a seeded random sweep of hard-ECC cases.

Each case draws a 2D or 3D shape (up to 1.5 M voxels, any row length, so
aligned and unaligned rows, full and partial column chunks), a value kind
(uint8, uniform float32, float32 with many ties, a wide normal field), a
threshold count H and a threshold kind (evenly spaced over the data, drawn
from the data's own values with repeats, unsorted and outside the data range,
or the data's quantiles), and compares the HIP result with the oracle bit for
bit.  Every case names itself on stdout before its GPU step.
"""

import numpy as np
import pytest

import oracle
from euler_characteristic_curves_amd import workloads as W
from tests.gpu_util import banner, need_gpu

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
