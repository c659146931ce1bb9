"""GPU parity of the batched hard ECC (B grids per call -> int64[B, H]).

Every row must equal the oracle's curve of that grid, bit for bit, for shared
thresholds ([H]) and per-grid thresholds ([B, H]).  Every case names itself
before its GPU step.
"""

import zlib

import numpy as np
import pytest

import oracle
from euler_characteristic_curves_amd import workloads as W
from tests.gpu_util import banner, need_gpu

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
