"""The soft forward and threshold backward against the float64 oracle within
the error bounds the ABI documents (include/ecc.h): float32 sigmoids of a few
ulps, plus |x| ulps where the exponent is formed in float32, and the
fixed-point combination of workgroup sums, all scaled by lambda |g_k| in the
backward.  The cases reach far past the 1e-4 / 1e-3 tolerance regime: upstream
gradients of a few thousand, lambda times the data range up to 2000 (lambda
up to 2e6 on the narrowest data), thresholds far outside the data, narrow and
wide value ranges.  Also a regression case for the fixed-point resolution: a
large lambda |g| on thresholds beyond the data, whose outputs are sums of
sigmoid tails."""

import numpy as np
import pytest

import oracle
from euler_characteristic_curves_amd import workloads as W
from tests.gpu_util import banner, soft_close
from tests.soft_bounds import soft_bounds, within

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def E():
    import euler_characteristic_curves_amd as E
    return E


def _cuda(*arrays):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrays]


def _case(rng):
    nd = int(rng.integers(2, 4))
    while True:
        dims = ([int(rng.integers(1, 30))] if nd == 3 else []) + [int(rng.integers(1, 100)),
                                                                   int(rng.integers(1, 300))]
        if np.prod(dims) <= 30_000:
            break
    shape = tuple(dims)
    kind = str(rng.choice(["uniform", "ties", "normal", "scaled"]))
    if kind == "uniform":
        g = rng.random(shape, dtype=np.float32)
    elif kind == "ties":
        g = (np.round(rng.random(shape) * 8) / 8).astype(np.float32)
    elif kind == "normal":
        g = rng.standard_normal(shape).astype(np.float32)
    else:
        g = (rng.random(shape) * float(rng.choice([1e-3, 1e3, 1e6]))).astype(np.float32)
    lo, hi = float(g.min()), float(g.max())
    span = hi - lo if hi > lo else 1.0
    H = int(rng.choice([1, 7, 64, 256, 300]))
    lam = float(np.float32(float(rng.choice([0.5, 5.0, 50.0, 500.0, 2000.0])) / span))
    tk = str(rng.choice(["linspace", "wide", "unsorted", "dups"]))
    if tk == "linspace":
        tau = W.tau_linspace(lo - 0.05 * span, hi + 0.05 * span, H)
    elif tk == "wide":
        tau = W.tau_linspace(lo - 3 * span, hi + 3 * span, H)
    elif tk == "unsorted":
        tau = rng.uniform(lo - 0.2 * span, hi + 0.2 * span, size=H).astype(np.float32)
    else:
        tau = np.sort(rng.choice(np.unique(g), size=H)).astype(np.float32)
    gout = (rng.standard_normal(H) * float(rng.choice([1e-3, 1.0, 1e3]))).astype(np.float32)
    return g, tau, lam, gout, f"{shape} {kind} H={H} lam={lam:g} {tk}"


@pytest.mark.parametrize("seed", range(4))
def test_soft_within_documented_bounds(E, seed):
    rng = np.random.default_rng(6100 + seed)
    for i in range(8):
        g, tau, lam, gout, name = _case(rng)
        banner("soft bounds", seed, i, name)
        dg, dt, dgo = _cuda(g, tau, gout)
        fb, tb = soft_bounds(g, tau, lam, gout)
        f = E.ecc_soft_fwd(dg, dt, lam).cpu().numpy()
        bad = within(f, oracle.ecc_soft(g, tau, lam), fb)
        assert bad.size == 0, (name, "forward", bad[:5])
        b = E.ecc_soft_bwd_tau(dg, dt, lam, dgo).cpu().numpy()
        bad = within(b, oracle.ecc_soft_bwd_tau(g, tau, lam, gout), tb)
        assert bad.size == 0, (name, "dL/dtau", bad[:5])


def test_soft_bwd_tau_tails_at_large_scale(E):
    """lambda = 5e4 on values in [0, 1e-3) (50 over the data range), upstream
    gradients of a few thousand, thresholds up to three data ranges outside
    the data.  Outputs for thresholds outside the data are sums of sigmoid
    tails, scaled by lambda |g_k| ~ 1e8: with the combination's resolution
    set by the grid size (2^-43 here) they meet the 1e-3 absolute / 1e-4
    relative tolerance, where a fixed 2^-40 let the rounding of the
    workgroup sums alone exceed it for the larger g_k."""
    rng = np.random.default_rng(77)
    g = (rng.random((60, 300)) * 1e-3).astype(np.float32)
    tau = np.linspace(-3e-3, 4e-3, 256).astype(np.float32)
    lam = float(np.float32(5e4))
    gout = (2000.0 * rng.standard_normal(256)).astype(np.float32)
    banner("soft tails", g.shape, "lam", lam)
    dg, dt, dgo = _cuda(g, tau, gout)
    b = E.ecc_soft_bwd_tau(dg, dt, lam, dgo).cpu().numpy()
    want = oracle.ecc_soft_bwd_tau(g, tau, lam, gout)
    _, tb = soft_bounds(g, tau, lam, gout)
    assert within(b, want, tb).size == 0
    tails = np.nonzero((tau < g.min()) | (tau > g.max()))[0]
    bad, worst = soft_close(b[tails], want[tails])
    assert bad.size == 0, (tails[bad[:5]], worst)
