"""GPU parity of the batched calls (B grids of one shape per call).

Hard: every row of int64[B, H] must equal the oracle's curve of that grid, bit
for bit, for shared thresholds ([H]) and per-grid thresholds ([B, H]).  Soft:
every grid's forward, threshold gradient and grid gradient within the soft
tolerance of the oracle.  Every case names itself before its GPU step.
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


def _batched_gpu(E, g, tau):
    import torch
    out = E.ecc_hard_batched(_dev(g), _dev(np.asarray(tau, np.float32)))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _grids(rng, B, shape, dtype):
    full = (B,) + tuple(shape)
    if dtype == "u8":
        return rng.integers(0, 256, size=full, dtype=np.uint8)
    if dtype == "f32":
        return rng.random(full, dtype=np.float32)
    return rng.integers(0, 5, size=full).astype(np.float32)  # ties


def _check(E, g, tau, name):
    banner("batched", name, g.shape, g.dtype, "tau", np.shape(tau))
    got = _batched_gpu(E, g, tau)
    want = oracle.ecc_hard_batched(g, tau)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{name}: {len(bad)} mismatches, first (b, k) {bad[:5].tolist()}"
    return got


@pytest.mark.parametrize("shape", [(1, 1), (2, 3), (33, 100), (128, 128), (130, 257), (1, 1, 1), (3, 4, 5),
                                   (9, 17, 33), (2, 64, 70)])
@pytest.mark.parametrize("B", [1, 2, 5, 64])
@pytest.mark.parametrize("dtype", ["u8", "f32", "ties"])
def test_batched_shared_tau(E, shape, B, dtype):
    rng = np.random.default_rng(zlib.crc32(repr(("bs", shape, B, dtype)).encode()))
    g = _grids(rng, B, shape, dtype)
    tau = W.tau_integers(256) if dtype == "u8" else W.tau_linspace(float(g.min()), float(g.max()), 300)
    _check(E, g, tau, f"shared-{dtype}")


@pytest.mark.parametrize("shape", [(47, 61), (128, 128), (6, 20, 24)])
@pytest.mark.parametrize("B", [3, 40])
def test_batched_per_grid_tau(E, shape, B):
    rng = np.random.default_rng(zlib.crc32(repr(("bp", shape, B)).encode()))
    g = (rng.random((B,) + shape) * rng.uniform(0.5, 3.0, size=(B,) + (1,) * len(shape))).astype(np.float32)
    tau = np.stack([W.tau_linspace(float(x.min()), float(x.max()), 200) for x in g])
    got = _check(E, g, tau, "per-grid")
    assert np.all(got[:, -1] == 1)
    # uint8 grids with a different threshold window per grid
    gu = rng.integers(0, 256, size=(B,) + shape, dtype=np.uint8)
    tu = np.stack([np.linspace(b, 255 - b, 64) for b in range(B)]).astype(np.float32)
    _check(E, gu, tu, "per-grid-u8")


@pytest.mark.parametrize("H", [1, 3, 1024, 4096])
def test_batched_threshold_counts(E, H):
    rng = np.random.default_rng(200 + H)
    g = rng.random((7, 40, 70), dtype=np.float32)
    _check(E, g, W.tau_linspace(0, 1, H), f"H={H}")


def test_batched_matches_single_calls(E):
    """Rows of a batch equal separate single-grid calls (bit for bit)."""
    import torch
    rng = np.random.default_rng(210)
    g = rng.random((6, 12, 50, 60), dtype=np.float32)
    tau = W.tau_linspace(0, 1, 512)
    banner("batched vs single")
    rows = _batched_gpu(E, g, tau)
    for b in range(g.shape[0]):
        one = E.ecc_hard_3d(_dev(g[b]), _dev(tau))
        torch.cuda.synchronize()
        assert np.array_equal(rows[b], one.cpu().numpy())


def test_batched_more_than_one_launch(E):
    """70000 grids need two launches of at most 65535 grid rows; 16 distinct
    grids repeat through the batch, so each row must equal its prototype's."""
    rng = np.random.default_rng(220)
    proto = rng.integers(0, 256, size=(16, 3, 4), dtype=np.uint8)
    B = 70000
    g = proto[np.arange(B) % 16]
    tau = W.tau_integers(256)
    banner("batched 70000 u8 3x4")
    got = _batched_gpu(E, g, tau)
    want = oracle.ecc_hard_batched(proto, tau)
    assert np.array_equal(got, want[np.arange(B) % 16])


def test_batched_workspace_reuse(E):
    """The workspace is left zero-filled: repeated calls with one workspace agree,
    also when a large batch follows a small one and vice versa."""
    import torch
    rng = np.random.default_rng(230)
    big = rng.random((3, 300, 2049), dtype=np.float32)
    small = rng.random((500, 16, 16), dtype=np.float32)
    tau = W.tau_linspace(0, 1, 256)
    nb = max(E.workspace_bytes_batched(0, 3, 256), E.workspace_bytes_batched(0, 500, 256))
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    banner("batched workspace reuse")
    want_big = oracle.ecc_hard_batched(big, tau)
    want_small = oracle.ecc_hard_batched(small, tau)
    for _ in range(2):
        for g, want in ((big, want_big), (small, want_small)):
            out = E.ecc_hard_batched(_dev(g), _dev(tau), ws=ws)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), want)
    assert int(torch.count_nonzero(ws).item()) == 0


# ------------------------------------------------------------ soft batches

def _soft_batched_gpu(E, g, tau, lam, gout):
    import torch
    dg, dt, dgo = _dev(g), _dev(np.asarray(tau, np.float32)), _dev(np.asarray(gout, np.float32))
    f = E.ecc_soft_fwd_batched(dg, dt, lam)
    b = E.ecc_soft_bwd_tau_batched(dg, dt, lam, dgo)
    gg = E.ecc_soft_bwd_grid_batched(dg, dt, lam, dgo)
    torch.cuda.synchronize()
    return (f.cpu().numpy().astype(np.float64), b.cpu().numpy().astype(np.float64),
            gg.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("shape", [(31, 47), (128, 128), (3, 4, 5), (17, 19, 23)])
@pytest.mark.parametrize("B", [1, 3, 16])
@pytest.mark.parametrize("per_grid", [False, True])
def test_soft_batched(E, shape, B, per_grid):
    rng = np.random.default_rng(zlib.crc32(repr(("soft-b", shape, B, per_grid)).encode()))
    g = rng.random((B,) + shape, dtype=np.float32)
    if per_grid:
        tau = np.stack([W.tau_linspace(-0.1 * b, 1.0 + 0.05 * b, 128) for b in range(B)])
    else:
        tau = W.tau_linspace(-0.05, 1.05, 128)
    gout = rng.standard_normal((B, 128)).astype(np.float32)
    lam = 40.0
    banner("soft batched", shape, B, "per-grid" if per_grid else "shared")
    f, bt, gg = _soft_batched_gpu(E, g, tau, lam, gout)
    for b in range(B):
        tb = tau[b] if per_grid else tau
        bad, worst = soft_close(f[b], oracle.ecc_soft(g[b], tb, lam))
        assert bad.size == 0, ("fwd", b, worst)
        bad, worst = soft_close(bt[b], oracle.ecc_soft_bwd_tau(g[b], tb, lam, gout[b]))
        assert bad.size == 0, ("bwd_tau", b, worst)
        bad, worst = soft_close(gg[b].ravel(), oracle.ecc_soft_bwd_grid(g[b], tb, lam, gout[b]).ravel())
        assert bad.size == 0, ("bwd_grid", b, worst)


def test_soft_batched_matches_single_calls(E):
    """The grid gradient of a batch equals single calls bit for bit; the curves
    agree to float64 rounding of the workgroup sums."""
    import torch
    rng = np.random.default_rng(240)
    g = rng.random((5, 40, 41, 42), dtype=np.float32)
    tau = W.tau_linspace(0, 1, 256)
    gout = rng.standard_normal((5, 256)).astype(np.float32)
    banner("soft batched vs single")
    f, bt, gg = _soft_batched_gpu(E, g, tau, 50.0, gout)
    dt = _dev(tau)
    for b in range(5):
        dg, dgo = _dev(g[b]), _dev(gout[b])
        f1 = E.ecc_soft_fwd(dg, dt, 50.0)
        b1 = E.ecc_soft_bwd_tau(dg, dt, 50.0, dgo)
        g1 = E.ecc_soft_bwd_grid(dg, dt, 50.0, dgo)
        torch.cuda.synchronize()
        assert np.array_equal(gg[b], g1.cpu().numpy().astype(np.float64))
        assert np.max(np.abs(f[b] - f1.cpu().numpy())) <= 1e-6 * max(1.0, np.max(np.abs(f[b])))
        assert np.max(np.abs(bt[b] - b1.cpu().numpy())) <= 1e-6 * max(1.0, np.max(np.abs(bt[b])))


def test_soft_batched_more_than_one_launch(E):
    """70000 tiny grids (two launches); 8 distinct grids repeat through the batch."""
    rng = np.random.default_rng(250)
    proto = rng.random((8, 2, 3), dtype=np.float32)
    B = 70000
    g = proto[np.arange(B) % 8]
    tau = W.tau_linspace(0, 1, 16)
    gout = np.tile(rng.standard_normal((8, 16)).astype(np.float32), (B // 8, 1))
    banner("soft batched 70000 2x3")
    f, bt, gg = _soft_batched_gpu(E, g, tau, 20.0, gout)
    for p in range(8):
        rows = np.arange(p, B, 8)
        bad, worst = soft_close(f[rows].ravel(), np.tile(oracle.ecc_soft(proto[p], tau, 20.0), rows.size))
        assert bad.size == 0, worst
        want_b = oracle.ecc_soft_bwd_tau(proto[p], tau, 20.0, gout[p])
        bad, worst = soft_close(bt[rows].ravel(), np.tile(want_b, rows.size))
        assert bad.size == 0, worst
        want_g = oracle.ecc_soft_bwd_grid(proto[p], tau, 20.0, gout[p]).ravel()
        bad, worst = soft_close(gg[rows].reshape(rows.size, -1).ravel(), np.tile(want_g, rows.size))
        assert bad.size == 0, worst


def test_soft_batched_autograd(E):
    import torch
    rng = np.random.default_rng(260)
    B = 4
    g = _dev(rng.random((B, 18, 19, 20), dtype=np.float32)).requires_grad_(True)
    tau = torch.tensor(W.tau_linspace(0, 1, 48)).cuda().requires_grad_(True)
    w = rng.standard_normal((B, 48)).astype(np.float32)
    banner("soft batched autograd")
    s = E.soft_ecc_batched(g, tau, 30.0)
    assert tuple(s.shape) == (B, 48)
    (s * torch.from_numpy(w).cuda()).sum().backward()
    gn, tn = g.detach().cpu().numpy(), tau.detach().cpu().numpy()
    want_tau = sum(oracle.ecc_soft_bwd_tau(gn[b], tn, 30.0, w[b]) for b in range(B))
    bad, worst = soft_close(tau.grad.cpu().numpy(), want_tau)
    assert bad.size == 0, worst
    for b in range(B):
        bad, worst = soft_close(g.grad[b].cpu().numpy().ravel(),
                                oracle.ecc_soft_bwd_grid(gn[b], tn, 30.0, w[b]).ravel())
        assert bad.size == 0, (b, worst)
    # per-grid thresholds: their gradient keeps the batch dimension
    tau2 = torch.tensor(np.stack([W.tau_linspace(0, 1, 48)] * B)).cuda().requires_grad_(True)
    E.soft_ecc_batched(g.detach(), tau2, 30.0).sum().backward()
    assert tuple(tau2.grad.shape) == (B, 48)


# ------------------------------------------- shared thresholds, summed
@pytest.mark.parametrize("B", [1, 2, 63, 64, 65, 130, 200])
@pytest.mark.parametrize("shape", [(9, 11), (5, 6, 7)])
def test_soft_bwd_tau_shared(E, B, shape):
    """dL/dtau of thresholds shared by the batch, summed on the device (groups
    of 64 grids, then the groups): the sum of the oracle's per-grid values.
    Repeated calls give the same bits and leave the workspace zero."""
    import torch
    rng = np.random.default_rng(zlib.crc32(repr(("shared", B, shape)).encode()))
    g = rng.random((B,) + shape, dtype=np.float32)
    tau = W.tau_linspace(-0.05, 1.05, 96)
    gout = rng.standard_normal((B, 96)).astype(np.float32)
    lam = 35.0
    ws = torch.zeros(E.workspace_bytes_batched(2, B, 96), dtype=torch.uint8, device="cuda")
    banner("soft bwd tau shared", B, shape)
    dg, dt, dgo = _dev(g), _dev(tau), _dev(gout)
    a = E.ecc_soft_bwd_tau_shared(dg, dt, lam, dgo, ws=ws)
    b = E.ecc_soft_bwd_tau_shared(dg, dt, lam, dgo, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert int(torch.count_nonzero(ws).item()) == 0
    want = sum(oracle.ecc_soft_bwd_tau(g[i], tau, lam, gout[i]) for i in range(B))
    bad, worst = soft_close(a.cpu().numpy(), want)
    assert bad.size == 0, worst


def test_soft_bwd_tau_shared_more_than_one_launch(E):
    """70000 tiny grids (two launches, 1094 groups of 64) drawn from 4096
    distinct grids, each batch entry with its own upstream gradient.  The sum
    is linear in g, so the oracle's value is sum_p lambda A_p (sum of g_b over
    the entries b holding grid p), with lambda A_p = ecc_soft_bwd_tau(p, g = 1).
    (Repeating a few grids thousands of times would multiply one grid's
    float32 rounding by the repeat count, which is no property of the sum.)"""
    import torch
    rng = np.random.default_rng(251)
    P, B = 4096, 70000
    proto = rng.random((P, 2, 3), dtype=np.float32)
    which = rng.integers(0, P, B)
    g = proto[which]
    tau = W.tau_linspace(0, 1, 16)
    gout = rng.standard_normal((B, 16)).astype(np.float32)
    banner("soft bwd tau shared 70000")
    got = E.ecc_soft_bwd_tau_shared(_dev(g), _dev(tau), 20.0, _dev(gout))
    torch.cuda.synchronize()
    G = np.zeros((P, 16))
    np.add.at(G, which, gout.astype(np.float64))
    ones = np.ones(16, np.float32)
    want = sum(G[p] * oracle.ecc_soft_bwd_tau(proto[p], tau, 20.0, ones) for p in np.unique(which))
    bad, worst = soft_close(got.cpu().numpy(), want)
    assert bad.size == 0, worst


def test_soft_curves_repeat_bit_for_bit(E):
    """Workgroup sums are formed in a fixed order and combined in fixed point:
    repeated calls give identical bits (single grid and batch)."""
    import torch
    rng = np.random.default_rng(252)
    g = _dev(rng.random((48, 50, 52), dtype=np.float32))
    gb = _dev(rng.random((6, 20, 21, 22), dtype=np.float32))
    tau = _dev(W.tau_linspace(0, 1, 300))
    go = _dev(rng.standard_normal(300).astype(np.float32))
    gob = _dev(rng.standard_normal((6, 300)).astype(np.float32))
    banner("soft repeat bits")
    runs = []
    for _ in range(3):
        runs.append([E.ecc_soft_fwd(g, tau, 40.0), E.ecc_soft_bwd_tau(g, tau, 40.0, go),
                     E.ecc_soft_fwd_batched(gb, tau, 40.0), E.ecc_soft_bwd_tau_batched(gb, tau, 40.0, gob)])
    torch.cuda.synchronize()
    for r in runs[1:]:
        for x, y in zip(runs[0], r):
            assert torch.equal(x, y)
