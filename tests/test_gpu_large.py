"""Grids past 2^32 voxels (64-bit indexing on every path), checked against
closed forms.

A checkerboard (value a where the index sum is even, b > a where it is odd)
has no cell with two corners of value a: every edge joins the two colours,
and every square or cube contains an edge.  So below b the sublevel complex
is the N_a isolated a-voxels (chi = N_a), and from b on it is the whole box
(chi = 1).  The soft curve follows from the same split: the N_a vertices have
value a and every other cell value b, and the signs of all cells sum to
chi(box) = 1, so S_k = N_a s(lambda (tau_k - a)) + (1 - N_a) s(lambda (tau_k - b)).
Grids are built on the GPU; nothing here needs the oracle.  Every case names
itself before its GPU step.
"""

import math

import numpy as np
import pytest

from tests.gpu_util import banner, need_gpu, soft_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def E():
    need_gpu()
    import euler_characteristic_curves_amd as E
    return E


def _checkerboard(shape, dtype, a, b):
    import torch
    parity = None
    for ax, n in enumerate(shape):
        v = (torch.arange(n, device="cuda") % 2).to(torch.uint8)
        v = v.reshape([-1 if i == ax else 1 for i in range(len(shape))])
        parity = v if parity is None else parity ^ v
    g = torch.empty(shape, dtype=dtype, device="cuda")
    g.copy_(parity)  # 0 / 1, broadcast to the full shape
    return g.mul_(b - a).add_(a)


def _n_even(shape):
    """Voxels whose index sum is even."""
    n = math.prod(shape)
    odd_all = all(s % 2 == 1 for s in shape)
    return (n + 1) // 2 if odd_all else n // 2


@pytest.mark.timeout(300)
def test_hard_2d_u8_past_2_32(E):
    import torch
    shape = (65537, 65539)  # 4.295e9 voxels, odd sides
    banner("large hard 2D u8", shape)
    g = _checkerboard(shape, torch.uint8, 0, 255)
    tau = torch.tensor([-1.0, 0.0, 100.0, 254.0, 255.0, 300.0], device="cuda")
    got = E.ecc_hard_2d(g, tau).cpu().tolist()
    del g
    torch.cuda.empty_cache()
    na = _n_even(shape)
    assert got == [0, na, na, na, 1, 1]


@pytest.mark.timeout(300)
def test_hard_3d_f32_past_2_32(E):
    import torch
    shape = (1025, 2048, 2049)  # 4.301e9 voxels, 17 GB
    banner("large hard 3D f32", shape)
    g = _checkerboard(shape, torch.float32, 0.0, 1.0)
    tau = torch.tensor([-1.0, 0.0, 0.5, 1.0, 2.0], device="cuda")
    got = E.ecc_hard_3d(g, tau).cpu().tolist()
    na = _n_even(shape)
    assert got == [0, na, na, 1, 1]
    # the soft curve of the same grid
    banner("large soft 3D f32", shape)
    lam = 8.0
    taus = np.array([-0.5, 0.0, 0.25, 0.5, 1.0, 1.5], np.float32)
    s = E.ecc_soft_fwd(g, torch.from_numpy(taus).cuda(), lam).cpu().numpy().astype(np.float64)
    del g
    torch.cuda.empty_cache()

    def sig(x):
        return 1.0 / (1.0 + math.exp(-x))
    want = np.array([na * sig(lam * float(t)) + (1 - na) * sig(lam * (float(t) - 1.0)) for t in taus])
    bad, worst = soft_close(s, want)
    assert bad.size == 0, (s, want, worst)


@pytest.mark.timeout(300)
def test_hard_batched_past_2_32(E):
    """1025 grids of 2048 x 2049 u8 (4.301e9 voxels in all): grid b is a
    checkerboard of values (b % 7, 200), so each row of the result has its own
    step position."""
    import torch
    B, ny, nx = 1025, 2048, 2049
    banner("large batched u8", (B, ny, nx))
    base = _checkerboard((ny, nx), torch.uint8, 0, 200)
    lo = (torch.arange(B, device="cuda") % 7).to(torch.uint8).reshape(B, 1, 1)
    g = torch.where(base.unsqueeze(0) == 0, lo, base.unsqueeze(0))
    tau = torch.arange(256, dtype=torch.float32, device="cuda")
    got = E.ecc_hard_batched(g, tau).cpu().numpy()
    del g, base
    torch.cuda.empty_cache()
    na = _n_even((ny, nx))
    k = np.arange(256)
    for b in (0, 1, 6, 7, 500, 1023, 1024):
        want = np.where(k < b % 7, 0, np.where(k < 200, na, 1))
        assert np.array_equal(got[b], want), b
