"""GPU parity of the directional heights and the single/multi-direction curves.

Heights f_d = X + alpha_d <u_d, p> must equal the oracle's float32 values bit
for bit, so the hard curves of f_d are bit-exact too.  The soft curves and all
gradients (grid, directions, scales, thresholds) must be within the soft
tolerance of the float64 oracle; the direction and scale gradients, sums over
the whole grid, also get 1e-5 of their magnitude (the same sums of |terms|),
which covers float32 rounding where terms of both signs cancel.  Every case
names itself before its GPU step.
"""

import zlib

import numpy as np
import pytest

import oracle
from euler_characteristic_curves_amd import workloads as W
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


def _case(shape, D, seed, with_inf=False):
    rng = np.random.default_rng(seed)
    X = rng.random(shape, dtype=np.float32)
    if with_inf:
        X[rng.random(shape) < 0.2] = np.inf
    U = rng.normal(size=(D, len(shape))).astype(np.float32)
    A = rng.uniform(-0.05, 0.05, size=D).astype(np.float32)
    return X, U, A


@pytest.mark.parametrize("shape", [(1, 1), (7, 5), (33, 1030), (16, 64), (1, 4), (1, 1, 1), (3, 7, 1100),
                                   (17, 19, 23), (5, 6, 128), (2, 3, 4)])
@pytest.mark.parametrize("D", [1, 3, 17])
def test_heights_bit_exact(E, shape, D):
    import torch
    X, U, A = _case(shape, D, zlib.crc32(repr(("h", shape, D)).encode()), with_inf=True)
    banner("heights", shape, D)
    f = E.ecc_height(_dev(X), _dev(U), _dev(A))
    torch.cuda.synchronize()
    got = f.cpu().numpy()
    want = oracle.height_values(X, U, A)
    assert got.shape == want.shape
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all(), np.argwhere(~same)[:5].tolist()


@pytest.mark.parametrize("shape", [(16, 49, 257), (9, 31, 259), (5, 17, 263), (3, 40, 299), (70, 257), (33, 1283)])
def test_heights_are_the_coordinates(E, shape):
    """Zero grid, alpha = 1 and unit directions: every height is a voxel
    coordinate, an exact float32.  Rows that are not a multiple of 4 voxels
    take the element-wise kernel, whose coordinates of 256 and more once
    came out wrong now and then (an integer-to-float conversion); the
    repeats give that a few chances to show."""
    import torch
    nd = len(shape)
    U = np.eye(nd, dtype=np.float32)
    A = np.ones(nd, np.float32)
    want = np.indices(shape).astype(np.float32)
    X = _dev(np.zeros(shape, np.float32))
    for rep in range(4):
        banner("height coordinates", shape, rep)
        got = E.ecc_height(X, _dev(U), _dev(A))
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        bad = np.argwhere(got != want)
        assert len(bad) == 0, (rep, bad[:5].tolist())


@pytest.mark.parametrize("nx", [257, 258, 261, 270, 283, 299])
def test_heights_bit_exact_rows_past_256(E, nx):
    import torch
    shape = (6, 23, nx)
    X, U, A = _case(shape, 7, zlib.crc32(repr(("h256", nx)).encode()))
    want = oracle.height_values(X, U, A)
    dX, dU, dA = _dev(X), _dev(U), _dev(A)
    for rep in range(3):
        banner("heights rows past 256", shape, rep)
        got = E.ecc_height(dX, dU, dA)
        torch.cuda.synchronize()
        bad = np.argwhere(got.cpu().numpy() != want)
        assert len(bad) == 0, (rep, bad[:5].tolist())


@pytest.mark.parametrize("shape", [(64, 96), (20, 24, 28)])
def test_hard_directional_bit_exact(E, shape):
    import torch
    X, U, A = _case(shape, 8, zlib.crc32(repr(("hd", shape)).encode()), with_inf=True)
    f = oracle.height_values(X, U, A)
    fin = f[np.isfinite(f)]
    tau = W.tau_linspace(float(fin.min()), float(fin.max()), 300)
    banner("hard directional", shape)
    got = E.ecc_hard_directional(_dev(X), _dev(U), _dev(A), _dev(tau))
    torch.cuda.synchronize()
    want = np.stack([oracle.ecc_hard(f[d], tau) for d in range(8)])
    assert np.array_equal(got.cpu().numpy(), want)


def test_hard_directional_frame_and_box(E):
    """The frame's (0, 1, 0) curve along x, and the box's step, on the GPU."""
    import torch
    X = np.zeros((7, 9), np.float32)
    X[2:5, 2:7] = np.inf
    tau = np.arange(-1, 10, dtype=np.float32)
    banner("directional frame")
    got = E.ecc_hard_directional(_dev(X), _dev(np.array([[0.0, 1.0]], np.float32)),
                                 _dev(np.array([1.0], np.float32)), _dev(tau))
    torch.cuda.synchronize()
    assert got.cpu().numpy()[0].tolist() == [0] + [1] * 7 + [0] * 3
    box = np.zeros((12, 13, 14), np.float32)
    U = np.random.default_rng(7).normal(size=(5, 3)).astype(np.float32)
    A = np.ones(5, np.float32)
    f = oracle.height_values(box, U, A)
    tau = np.linspace(-40, 40, 81).astype(np.float32)
    got = E.ecc_hard_directional(_dev(box), _dev(U), _dev(A), _dev(tau))
    torch.cuda.synchronize()
    want = np.stack([(tau >= f[d].min()).astype(np.int64) for d in range(5)])
    assert np.array_equal(got.cpu().numpy(), want)


def _moment_close(got, want, carried):
    """The soft tolerance of the result plus ``carried``: the error a result
    inherits from inputs that are themselves only within a tolerance."""
    got, want, carried = (np.asarray(v, np.float64).ravel() for v in (got, want, carried))
    tol = np.where(np.abs(want) >= 10, 1e-4 * np.abs(want), 1e-3) + carried
    err = np.abs(got - want)
    return np.nonzero(~(err <= tol))[0], float(np.max(err / tol)) if err.size else 0.0


def _carried_bounds(G, U, A):
    """Bounds on the errors of dL/du and dL/dalpha when each G[d](p) may be off
    by its soft tolerance t(p) = max(1e-3, 1e-4 |G[d](p)|): M[d, i] moves by at
    most sum_p t(p) |p_i|, so dL/du by |alpha_d| times that and dL/dalpha by
    sum_i |u_d,i| times that (the chain rule of height_bwd with every factor
    replaced by its magnitude)."""
    t = np.maximum(1e-3, 1e-4 * np.abs(np.asarray(G, np.float64)))
    _, bu, ba = oracle.height_bwd(t, np.abs(U), np.abs(A))
    return bu, ba


@pytest.mark.parametrize("shape", [(1, 1), (31, 47), (130, 70), (64, 128), (1, 4), (9, 17, 33), (40, 41, 42),
                                   (10, 12, 16), (3, 5, 4)])
@pytest.mark.parametrize("D", [1, 5])
def test_height_bwd(E, shape, D):
    import torch
    rng = np.random.default_rng(zlib.crc32(repr(("hb", shape, D)).encode()))
    G = rng.standard_normal((D,) + shape).astype(np.float32)
    U = rng.normal(size=(D, len(shape))).astype(np.float32)
    A = rng.uniform(-2, 2, size=D).astype(np.float32)
    banner("height bwd", shape, D)
    dG, dU, dA = _dev(G), _dev(U), _dev(A)
    gg, gd, ga = E.ecc_height_bwd(dG, dU, dA)
    gg2, gd2, ga2 = E.ecc_height_bwd(dG, dU, dA)
    torch.cuda.synchronize()
    wg, wd, wa = oracle.height_bwd(G, U, A)
    bad, worst = soft_close(gg.cpu().numpy().ravel(), wg.ravel())
    assert bad.size == 0, worst
    bad, worst = soft_close(gd.cpu().numpy().ravel(), wd.ravel())
    assert bad.size == 0, worst
    bad, worst = soft_close(ga.cpu().numpy().ravel(), wa.ravel())
    assert bad.size == 0, worst
    # deterministic: the same bits on a second call
    for a, b in ((gg, gg2), (gd, gd2), (ga, ga2)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("shape", [(48, 50), (40, 64), (20, 21, 22), (16, 20, 24)])
def test_soft_directional_forward_and_gradients(E, shape):
    """Soft curves of D directions and the gradients of all four inputs,
    through the autograd chain heights -> batched soft curves."""
    import torch
    D, H, lam = 4, 96, 30.0
    X, U, A = _case(shape, D, zlib.crc32(repr(("sd", shape)).encode()))
    tau = W.tau_linspace(-1.0, 2.0, H)
    w = np.random.default_rng(5).standard_normal((D, H)).astype(np.float32)
    dX = _dev(X).requires_grad_(True)
    dU = _dev(U).requires_grad_(True)
    dA = _dev(A).requires_grad_(True)
    dT = _dev(tau).requires_grad_(True)
    banner("soft directional", shape)
    S = E.soft_ecc_directional(dX, dU, dA, dT, lam)
    (S * _dev(w)).sum().backward()
    torch.cuda.synchronize()
    f = oracle.height_values(X, U, A)
    for d in range(D):
        bad, worst = soft_close(S[d].detach().cpu().numpy(), oracle.ecc_soft(f[d], tau, lam))
        assert bad.size == 0, ("fwd", d, worst)
    want_tau = sum(oracle.ecc_soft_bwd_tau(f[d], tau, lam, w[d]) for d in range(D))
    bad, worst = soft_close(dT.grad.cpu().numpy(), want_tau)
    assert bad.size == 0, ("tau", worst)
    G = np.stack([oracle.ecc_soft_bwd_grid(f[d], tau, lam, w[d]) for d in range(D)])
    wg, wd, wa = oracle.height_bwd(G, U, A)
    bu, ba = _carried_bounds(G, U, A)
    # dL/dX sums the D grid gradients, each within its own soft tolerance
    bx = np.maximum(1e-3, 1e-4 * np.abs(G)).sum(axis=0)
    bad, worst = _moment_close(dX.grad.cpu().numpy(), wg, bx)
    assert bad.size == 0, ("grid", worst)
    bad, worst = _moment_close(dU.grad.cpu().numpy(), wd, bu)
    assert bad.size == 0, ("dirs", worst)
    bad, worst = _moment_close(dA.grad.cpu().numpy(), wa, ba)
    assert bad.size == 0, ("alpha", worst)
