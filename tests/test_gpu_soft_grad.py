"""GPU parity of the soft ECC gradient with respect to the grid.

The HIP kernel (through the C ABI) against the float64 oracle, voxel by voxel:
within 1e-4 relative where |value| >= 10, else 1e-3 absolute (the soft ECC
tolerance).  At the 256^3 soft workload the oracle runs on z-slabs in worker
processes and every voxel is compared; the whole result is also checked
against the sum rule sum_p dL/dX(p) = -sum_k dL/dtau_k.  Every case names itself before its GPU step.
"""

import zlib

import numpy as np
import pytest

import oracle
from euler_characteristic_curves_amd import workloads as W
from tests import slabs
from tests.gpu_util import banner, need_gpu, soft_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def E():
    need_gpu()
    import euler_characteristic_curves_amd as E
    return E


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _grad_gpu(E, g, tau, lam, gout):
    import torch
    r = E.ecc_soft_bwd_grid(_dev(g), _dev(np.asarray(tau, np.float32)), lam,
                            _dev(np.asarray(gout, np.float32)))
    torch.cuda.synchronize()
    return r.cpu().numpy().astype(np.float64)


def _check(E, g, tau, lam, gout, name):
    banner("soft grad", name, g.shape, "H=%d" % len(tau), "lam=%g" % lam)
    got = _grad_gpu(E, g, tau, lam, gout)
    assert got.shape == g.shape
    want = oracle.ecc_soft_bwd_grid(g, tau, lam, gout)
    bad, worst = soft_close(got.ravel(), want.ravel())
    assert bad.size == 0, (name, np.unravel_index(bad[:5], g.shape), got.ravel()[bad[:5]],
                           want.ravel()[bad[:5]], worst)
    return got, want


@pytest.mark.parametrize("shape", [(1, 1), (1, 9), (13, 1), (31, 47), (200, 300), (1, 1, 1), (3, 4, 5),
                                   (1, 30, 70), (17, 19, 23), (40, 40, 40), (2, 1, 700), (5, 3, 257)])
@pytest.mark.parametrize("lam", [0.5, 50.0, 2000.0])
def test_soft_grad_small(E, shape, lam):
    rng = np.random.default_rng(zlib.crc32(repr(("grad", shape, lam)).encode()))
    g = rng.random(shape, dtype=np.float32)
    tau = W.tau_linspace(-0.05, 1.05, 256 if lam != 2000.0 else 301)
    gout = rng.standard_normal(tau.size).astype(np.float32)
    _check(E, g, tau, lam, gout, "uniform")


@pytest.mark.parametrize("shape", [(47, 61), (21, 33, 17)])
def test_soft_grad_ties(E, shape):
    """Plateaus: most cells have tied corners, so the first-index rule decides c(p)."""
    rng = np.random.default_rng(zlib.crc32(repr(("ties", shape)).encode()))
    g = (rng.integers(0, 9, shape) / 8).astype(np.float32)
    for tau, lam in [(np.array([0.5], np.float32), 10.0),
                     (rng.permutation(W.tau_linspace(-1, 2, 777)), 30.0),
                     (W.tau_linspace(0, 1, 1000), 1e4),
                     (np.array([0.0, 0.125, 0.25, 0.375, 0.5, 0.625, 0.75, 0.875, 1.0], np.float32), 40.0)]:
        gout = rng.standard_normal(tau.size).astype(np.float32)
        _check(E, g, tau, lam, gout, "ties")
    # a constant grid: everything goes to the last voxel
    c = np.full(shape, 0.25, np.float32)
    tau = W.tau_linspace(0, 1, 64)
    gout = rng.standard_normal(64).astype(np.float32)
    got, want = _check(E, c, tau, 20.0, gout, "constant")
    assert np.count_nonzero(got) <= 1 and np.count_nonzero(want) == 1


def test_soft_grad_direct_exponent_paths(E):
    """Threshold spans that leave the factored form, and upstream gradients of
    1e8 with both signs, whose terms cancel to below float32 resolution at
    voxels near a zero of h: those take the float64 path.  The soft tolerance
    applies unchanged."""
    rng = np.random.default_rng(41)
    g = rng.random((19, 23, 29), dtype=np.float32)
    cases = [
        (np.array([-1e30, -5, 0.25, 0.25, 0.5, 7, 1e30], np.float32), 5.0,
         rng.standard_normal(7).astype(np.float32)),
        (W.tau_linspace(-3, 4, 200), 60.0, rng.standard_normal(200).astype(np.float32)),
        (W.tau_linspace(0, 1, 100), 50.0, (rng.standard_normal(100) * 1e8).astype(np.float32)),
        (W.tau_linspace(-3, 4, 200), 60.0, (rng.standard_normal(200) * 1e8).astype(np.float32)),
    ]
    for tau, lam, gout in cases:
        _check(E, g, tau, lam, gout, "direct/large g")


def test_soft_grad_cancellation_and_far_values(E):
    """Voxels far above every threshold (the float factor would overflow),
    far below (it underflows), tiny and huge upstream gradients, and a large
    lambda with alternating-sign gradients, where h(v) cancels."""
    rng = np.random.default_rng(47)
    shape = (13, 17, 21)
    g = rng.random(shape, dtype=np.float32)
    g[:4] *= 40.0            # far above tau in [0, 1]
    g[-4:] -= 40.0           # far below
    tau = W.tau_linspace(0, 1, 64)
    # The oracle adds each cell type's share separately; where they cancel
    # (c(p) = 0) its float64 residue is about 2^-53 lambda sum_k |g_k| s(1 - s),
    # so upstream gradients stay at or below 1e8 for the 1e-3 absolute tolerance.
    for scale in (1e-30, 1.0, 1e6, 1e8):
        gout = (rng.standard_normal(64) * scale).astype(np.float32)
        _check(E, g, tau, 50.0, gout, f"far values, |g|~{scale:g}")
    u = rng.random(shape, dtype=np.float32)
    alt = np.where(np.arange(300) % 2 == 0, 1.0, -1.0).astype(np.float32)
    _check(E, u, W.tau_linspace(0, 1, 300), 2000.0, alt, "alternating g, lambda 2000")
    _check(E, u, W.tau_linspace(0, 1, 300), 2000.0, alt * np.float32(1e7), "alternating g x 1e7")


@pytest.mark.parametrize("H", [1, 2, 3, 255, 4096, 8192])
def test_soft_grad_threshold_counts(E, H):
    rng = np.random.default_rng(100 + H)
    g = rng.random((11 if H <= 4096 else 5, 13, 70), dtype=np.float32)
    tau = W.tau_linspace(0, 1, H)
    gout = rng.standard_normal(H).astype(np.float32)
    _check(E, g, tau, 25.0, gout, f"H={H}")


def test_soft_grad_smooth_field(E):
    """A Gaussian random field: few voxels with c != 0, so the queues rarely fill."""
    g = W.gaussian_random_field((48, 50, 52), 3.0, 5)
    tau = W.tau_linspace(float(g.min()), float(g.max()), 256)
    gout = np.random.default_rng(6).standard_normal(256).astype(np.float32)
    got, _ = _check(E, g, tau, 50.0, gout, "grf")
    assert np.count_nonzero(got) < 0.1 * g.size


def test_soft_grad_sum_rule_and_repeat(E):
    """sum_p dL/dX(p) = -sum_k dL/dtau_k on the GPU's own two outputs; repeated
    calls give identical bits (each voxel is written once, no atomics)."""
    rng = np.random.default_rng(43)
    g = rng.random((64, 64, 64), dtype=np.float32)
    tau = W.tau_linspace(0, 1, 256)
    gout = rng.standard_normal(256).astype(np.float32)
    banner("soft grad sum rule 64^3")
    a = _grad_gpu(E, g, tau, 50.0, gout)
    b = _grad_gpu(E, g, tau, 50.0, gout)
    assert np.array_equal(a, b)
    import torch
    gt = E.ecc_soft_bwd_tau(_dev(g), _dev(tau), 50.0, _dev(gout))
    torch.cuda.synchronize()
    gt = gt.cpu().numpy().astype(np.float64)
    assert abs(a.sum() + gt.sum()) <= 1e-5 * np.abs(a).sum() + 1e-3


@pytest.mark.timeout(600)
def test_config_256cube_soft_grad(E):
    """The 256^3 soft workload: every voxel against the whole-grid oracle,
    which runs on z-slabs in spawned CPU worker processes (tests/slabs.py),
    plus the sum rule against the GPU's own dL/dtau."""
    import torch
    g, tau, extra = W.make_workload("c5_256cube_soft")
    lam, gout = extra["lam"], extra["grad_out"]
    banner("soft grad c5")
    got = _grad_gpu(E, g, tau, lam, gout)
    banner("soft grad c5: oracle on z-slabs in worker processes")
    want = slabs.workload_grad("c5_256cube_soft")
    bad, worst = soft_close(got.ravel(), want.ravel())
    assert bad.size == 0, (np.unravel_index(bad[:5], g.shape), got.ravel()[bad[:5]], want.ravel()[bad[:5]], worst)
    gt = E.ecc_soft_bwd_tau(_dev(g), _dev(tau), lam, _dev(gout))
    torch.cuda.synchronize()
    gt = gt.cpu().numpy().astype(np.float64)
    assert abs(got.sum() + gt.sum()) <= 1e-5 * np.abs(got).sum() + 1e-2


def test_autograd_grid_and_tau(E):
    import torch
    rng = np.random.default_rng(45)
    g = _dev(rng.random((20, 21, 22), dtype=np.float32)).requires_grad_(True)
    tau = torch.tensor(W.tau_linspace(0, 1, 64)).cuda().requires_grad_(True)
    w = rng.standard_normal(64).astype(np.float32)
    banner("autograd grid+tau")
    s = E.soft_ecc(g, tau, 25.0)
    (s * torch.from_numpy(w).cuda()).sum().backward()
    gn, tn = g.detach().cpu().numpy(), tau.detach().cpu().numpy()
    bad, worst = soft_close(g.grad.cpu().numpy().ravel(), oracle.ecc_soft_bwd_grid(gn, tn, 25.0, w).ravel())
    assert bad.size == 0, worst
    bad, worst = soft_close(tau.grad.cpu().numpy(), oracle.ecc_soft_bwd_tau(gn, tn, 25.0, w))
    assert bad.size == 0, worst
    # grid only: tau's gradient is not computed
    g.grad = None
    tau2 = tau.detach()
    E.soft_ecc(g, tau2, 25.0).sum().backward()
    assert g.grad is not None and g.grad.shape == g.shape
