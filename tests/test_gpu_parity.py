"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Hard ECC must match bit for bit (int64).  Soft ECC forward and backward must
be within 1e-4 relative of the float64 oracle where |value| >= 10, else 1e-3
absolute.  Every case names itself on stdout before its GPU step.
"""

import zlib

import numpy as np
import pytest

import oracle
from euler_characteristic_curves_amd import workloads as W
from tests import golden_curves
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


def _hard_gpu(E, g, tau):
    import torch
    out = E.ecc_hard(_dev(g), _dev(np.asarray(tau, np.float32)))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_hard(E, g, tau, name):
    banner("hard", name, g.shape, g.dtype, "H=%d" % len(tau))
    got = _hard_gpu(E, g, tau)
    want = oracle.ecc_hard(g, tau)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{name}: {bad.size} mismatches, first k={bad[:5]} got={got[bad[:5]]} want={want[bad[:5]]}"


def _taus(rng, g, H, kind):
    lo, hi = float(np.min(g)), float(np.max(g))
    if kind == "linspace":
        return W.tau_linspace(lo, hi, H)
    if kind == "dups":
        t = np.sort(rng.choice(np.unique(g.astype(np.float32)), size=H)).astype(np.float32)
        return t
    if kind == "unsorted":
        return rng.uniform(lo - 0.1 * abs(lo) - 1, hi + 1, size=H).astype(np.float32)
    raise ValueError(kind)


SHAPES_2D = [(1, 1), (1, 7), (7, 1), (5, 13), (33, 100), (64, 1024), (130, 257), (17, 1500),
             (300, 2049), (256, 4096), (1000, 129), (3, 5000)]
SHAPES_3D = [(1, 1, 1), (1, 5, 7), (2, 3, 4), (9, 17, 33), (20, 30, 300), (64, 64, 64), (5, 300, 257),
             (40, 1, 1), (3, 2, 1100), (70, 9, 260), (6, 7, 768)]


@pytest.mark.parametrize("shape", SHAPES_2D + SHAPES_3D)
@pytest.mark.parametrize("dtype", ["u8", "f32", "f32ties"])
def test_hard_random_shapes(E, shape, dtype):
    rng = np.random.default_rng(zlib.crc32(repr((shape, dtype)).encode()))
    if dtype == "u8":
        g = rng.integers(0, 256, size=shape, dtype=np.uint8)
    elif dtype == "f32":
        g = rng.random(shape, dtype=np.float32)
    else:
        g = rng.integers(0, 6, size=shape).astype(np.float32)
    for H, kind in [(1, "linspace"), (2, "linspace"), (255, "linspace"), (256, "dups"), (97, "unsorted"),
                    (1024, "linspace")]:
        _check_hard(E, g, _taus(rng, g, H, kind), f"{dtype}-{kind}")


@pytest.mark.parametrize("ntiles", [1, 2, 7, 8, 9, 15, 16, 17, 23, 64, 65, 127, 300])
def test_hard_tile_counts_around_xcd_split(E, ntiles):
    """Small grids launch one workgroup per tile; below 8 workgroups the tiles are
    strided, from 8 up every XCD takes a contiguous share.  Tile counts around
    multiples of 8 (with uneven shares) must still cover every tile once."""
    rng = np.random.default_rng(zlib.crc32(repr(("tiles", ntiles)).encode()))
    # 2D float: a 256-column chunk by four one-row wave tiles per tile
    g = rng.random((4 * ntiles, 256), dtype=np.float32)
    _check_hard(E, g, W.tau_linspace(0.0, 1.0, 200), f"tiles2d-{ntiles}")
    # 2D uint8: a 1024-column chunk per tile
    g8 = rng.integers(0, 256, size=(4 * ntiles, 1024), dtype=np.uint8)
    _check_hard(E, g8, W.tau_integers(256), f"tiles2d-u8-{ntiles}")
    # 3D float: a 256-column chunk, 32 rows, two planes per tile
    g3 = rng.random((2 * ntiles, 32, 256), dtype=np.float32)
    _check_hard(E, g3, W.tau_linspace(0.0, 1.0, 64), f"tiles3d-{ntiles}")


@pytest.mark.parametrize("nx", [4, 16, 32, 64, 124, 128, 252, 260, 528, 1008, 1040, 1552])
@pytest.mark.parametrize("dtype", ["u8", "f32", "f32ties"])
def test_hard_aligned_partial_chunks(E, nx, dtype):
    """Aligned rows whose last column chunk ends inside the row (narrow grids,
    ragged right edges): lanes past the row end carry no cells."""
    if dtype == "u8" and nx % 16:
        nx = nx + (16 - nx % 16)  # keep u8 rows 16-byte aligned too
    rng = np.random.default_rng(zlib.crc32(repr(("partial", nx, dtype)).encode()))
    for ny in (1, 2, 7, 130):
        if dtype == "u8":
            g = rng.integers(0, 256, size=(ny, nx), dtype=np.uint8)
            tau = W.tau_integers(256)
        elif dtype == "f32":
            g = rng.random((ny, nx), dtype=np.float32)
            tau = W.tau_linspace(0.0, 1.0, 300)
        else:
            g = rng.integers(0, 4, size=(ny, nx)).astype(np.float32)
            tau = np.array([-1, 0, 0.5, 1, 2, 3, 4], np.float32)
        _check_hard(E, g, tau, f"partial-{dtype}-{ny}x{nx}")


@pytest.mark.parametrize("H", [1, 3, 511, 512, 513, 2048, 4096, 8192])
def test_hard_threshold_counts(E, H):
    rng = np.random.default_rng(H)
    g2 = rng.random((77, 333), dtype=np.float32)
    g3 = rng.random((11, 23, 45), dtype=np.float32)
    for g in (g2, g3):
        _check_hard(E, g, W.tau_linspace(0.0, 1.0, H), f"H{H}")
        _check_hard(E, g, _taus(rng, g, H, "unsorted"), f"H{H}-unsorted")
    gu = rng.integers(0, 256, (45, 1000), dtype=np.uint8)
    _check_hard(E, gu, (np.arange(H) * 255.0 / max(H - 1, 1)).astype(np.float32), f"u8-H{H}")


def test_hard_threshold_spacings_3d(E):
    """Float 3D binning for evenly spaced, quantile-spaced, heavily clustered and
    repeated thresholds (the kernel bins by a one-per-bucket table, a small
    per-bucket scan, or a binary search, depending on the spacing)."""
    g = W.gaussian_random_field((33, 40, 300), 2.0, 77)
    gmin, gmax = float(g.min()), float(g.max())
    flat = np.sort(g.ravel()[::13].astype(np.float64))
    cases = {
        "linspace": W.tau_linspace(gmin, gmax, 512),
        "quantiles": np.quantile(flat, np.linspace(0, 1, 512)).astype(np.float32),
        "cluster": np.sort(np.concatenate([[gmin, gmax], np.linspace(0.0, 1e-3, 400)])).astype(np.float32),
        "repeats": np.sort(np.repeat(np.linspace(gmin, gmax, 37), 7)).astype(np.float32),
        "wide": np.sort(np.concatenate([[-1e30, 1e30], np.linspace(gmin, gmax, 100)])).astype(np.float32),
    }
    for name, tau in cases.items():
        _check_hard(E, g, tau, "3d-" + name)


def test_hard_bucket_map_offsets_3d(E):
    """Float 3D binning where the bucket map is least comfortable: values far
    from zero in a narrow band (the map's offset is large next to its range),
    a range of a few ulps, values at the bucket boundaries of linspace
    thresholds (threshold values themselves and their float neighbours), and
    magnitudes near the float limits."""
    rng = np.random.default_rng(41)
    shape = (9, 21, 300)
    cases = []
    for offset, width in ((1e6, 1.0), (-3e7, 64.0), (1.0, 1e-6), (5e4, 1e-2), (-1e-30, 1e-33)):
        g = (offset + width * rng.random(shape)).astype(np.float32)
        vals = np.unique(g)
        # distinct thresholds: every value of a coarse band, else evenly spaced
        tau = vals if vals.size <= 300 else W.tau_linspace(float(vals[0]), float(vals[-1]), 257)
        cases.append((f"band-{offset:g}", g, tau.astype(np.float32)))
    # a range of a few ulps: many grid values equal, thresholds nearly equal
    base = np.float32(1.5)
    steps = np.nextafter(np.float32(base), np.float32(2), dtype=np.float32)
    ulps = np.array([base, steps, np.nextafter(steps, np.float32(2), dtype=np.float32)], np.float32)
    g = rng.choice(ulps, size=shape).astype(np.float32)
    cases.append(("ulps", g, np.sort(rng.choice(ulps, 5)).astype(np.float32)))
    # grid values on the thresholds and one ulp either side of them
    tau = W.tau_linspace(-2.0, 3.0, 300)
    near = np.concatenate([tau, np.nextafter(tau, np.float32(-np.inf)), np.nextafter(tau, np.float32(np.inf))])
    g = rng.choice(near.astype(np.float32), size=shape).astype(np.float32)
    cases.append(("on-thresholds", g, tau))
    g = (rng.standard_normal(shape) * 1e37).astype(np.float32)
    cases.append(("huge", g, W.tau_linspace(float(g.min()), float(g.max()), 200)))
    for name, g, tau in cases:
        _check_hard(E, g, tau, "3d-map-" + name)


def test_hard_special_values(E):
    rng = np.random.default_rng(5)
    specials = np.array([-0.0, 0.0, 1e-45, -1e-45, 1e-38, np.inf, -np.inf, 1.0, -1.0, 3e38], np.float32)
    for shape in [(19, 37), (6, 7, 21)]:
        g = rng.choice(specials, size=shape).astype(np.float32)
        tau = np.array([-np.inf, -3e38, -1.0, -1e-45, -0.0, 0.0, 1e-45, 1e-38, 1.0, 3e38, np.inf],
                       np.float32)
        _check_hard(E, g, tau, "specials")
        _check_hard(E, g, rng.permutation(tau), "specials-unsorted")


def test_hard_uint8_threshold_edges(E):
    rng = np.random.default_rng(9)
    g = rng.integers(0, 256, (123, 517), dtype=np.uint8)
    tau = np.array([-np.inf, -1, -0.5, 0, 0.5, 1, 254.5, 254.99, 255, 255.5, 1e9, np.inf, 7, 3],
                   np.float32)
    _check_hard(E, g, tau, "u8-edges")
    g3 = rng.integers(0, 256, (7, 33, 129), dtype=np.uint8)
    _check_hard(E, g3, tau, "u8-edges-3d")


def test_hard_misaligned_views(E):
    import torch
    rng = np.random.default_rng(13)
    for dtype, shape in [(np.float32, (64, 256)), (np.uint8, (64, 1024)), (np.float32, (8, 16, 256)),
                         (np.uint8, (8, 16, 512))]:
        g = (rng.random(shape) * 50).astype(dtype)
        flat = np.concatenate([np.zeros(1, dtype), g.ravel()])
        t = torch.from_numpy(flat).cuda()[1:].view(*shape)
        tau = W.tau_linspace(0, 50, 300)
        banner("hard misaligned", shape, dtype)
        got = E.ecc_hard(t, _dev(tau)).cpu().numpy()
        assert np.array_equal(got, oracle.ecc_hard(g, tau))


def test_hard_repeat_and_metamorphic(E):
    rng = np.random.default_rng(17)
    g = rng.integers(0, 256, (512, 2048), dtype=np.uint8)
    tau = W.tau_integers(256)
    banner("hard repeat", g.shape)
    first = _hard_gpu(E, g, tau)
    assert np.array_equal(first, oracle.ecc_hard(g, tau))
    for _ in range(5):
        assert np.array_equal(_hard_gpu(E, g, tau), first)
    for h in (g.T, g[::-1], g[:, ::-1]):
        assert np.array_equal(_hard_gpu(E, np.ascontiguousarray(h), tau), first)
    assert np.array_equal(_hard_gpu(E, g.astype(np.float32), tau), first)
    g3 = rng.random((30, 40, 50), dtype=np.float32)
    t3 = W.tau_linspace(0, 1, 512)
    base = _hard_gpu(E, g3, t3)
    for perm in [(0, 2, 1), (2, 1, 0), (1, 0, 2)]:
        assert np.array_equal(_hard_gpu(E, np.ascontiguousarray(g3.transpose(perm)), t3), base)


def test_hard_inclusion_exclusion(E):
    """chi(A u B) = chi(A) + chi(B) - chi(A n B) for two z-slabs sharing one plane."""
    rng = np.random.default_rng(19)
    g = rng.random((37, 50, 260), dtype=np.float32)
    tau = W.tau_linspace(0, 1, 200)
    banner("hard inclusion-exclusion", g.shape)
    whole = _hard_gpu(E, g, tau)
    m = 20
    top = _hard_gpu(E, g[: m + 1], tau)
    bot = _hard_gpu(E, g[m:], tau)
    mid = _hard_gpu(E, g[m], tau)
    assert np.array_equal(whole, top + bot - mid)


# ---------------------------------------------------------------- configs
def test_config_128sq(E):
    g, tau, _ = W.make_workload("c1_128sq_f32")
    _check_hard(E, g, tau, "c1")


def test_config_1024sq_grf(E):
    g, tau, _ = W.make_workload("c2_1024sq_f32_grf")
    _check_hard(E, g, tau, "c2")


@pytest.mark.timeout(300)
def test_config_8192sq_u8(E):
    g, tau, _ = W.make_workload("c3_8192sq_u8")
    _check_hard(E, g, tau, "c3")


def _check_whole_curve(E, name, timeout_note):
    """All H outputs against the oracle's stored whole curve (tests/golden/
    config_curves.json); when the regenerated input differs from the recorded
    bytes (the Gaussian random field goes through a floating-point FFT), the
    oracle is run here instead."""
    import torch
    g, tau, _ = W.make_workload(name)
    rec = golden_curves.load(name)
    if golden_curves.same_inputs(rec, g, tau):
        want = np.array(rec["ecc"], np.int64)
    else:
        banner("input differs from the recorded one: running the oracle", name, timeout_note)
        want = oracle.ecc_hard(g, tau)
    banner("hard", name, g.shape, g.dtype, "H=%d" % len(tau))
    got = E.ecc_hard(_dev(g), _dev(tau))
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{name}: {bad.size} mismatches, first k={bad[:5]} got={got[bad[:5]]} want={want[bad[:5]]}"
    assert got[-1] == 1
    return got


@pytest.mark.timeout(300)
def test_config_512cube_grf(E):
    _check_whole_curve(E, "c4a_512cube_f32_grf", "about 30 s")


@pytest.mark.timeout(600)
def test_config_1024cube(E):
    _check_whole_curve(E, "c4b_1024cube_f32", "several minutes")


# ------------------------------------------------------------------- soft
def _soft_gpu(E, g, tau, lam, gout=None):
    import torch
    dg, dt = _dev(g), _dev(np.asarray(tau, np.float32))
    if gout is None:
        r = E.ecc_soft_fwd(dg, dt, lam)
    else:
        r = E.ecc_soft_bwd_tau(dg, dt, lam, _dev(np.asarray(gout, np.float32)))
    torch.cuda.synchronize()
    return r.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("shape", [(1, 1), (1, 9), (13, 1), (31, 47), (200, 300), (1, 1, 1), (3, 4, 5),
                                   (17, 19, 23), (40, 40, 40), (2, 1, 700)])
@pytest.mark.parametrize("lam", [0.5, 50.0, 2000.0])
def test_soft_small(E, shape, lam):
    rng = np.random.default_rng(zlib.crc32(repr((shape, lam)).encode()))
    g = rng.random(shape, dtype=np.float32)
    tau = W.tau_linspace(-0.05, 1.05, 256 if lam != 2000.0 else 300)
    gout = rng.standard_normal(tau.size).astype(np.float32)
    banner("soft fwd", shape, lam)
    f = _soft_gpu(E, g, tau, lam)
    bad, worst = soft_close(f, oracle.ecc_soft(g, tau, lam))
    assert bad.size == 0, (bad[:5], worst)
    banner("soft bwd", shape, lam)
    b = _soft_gpu(E, g, tau, lam, gout)
    bad, worst = soft_close(b, oracle.ecc_soft_bwd_tau(g, tau, lam, gout))
    assert bad.size == 0, (bad[:5], worst)


def test_soft_ties_and_odd_thresholds(E):
    rng = np.random.default_rng(23)
    g = (rng.integers(0, 9, (21, 33, 17)) / 8).astype(np.float32)
    for tau, lam in [(np.array([0.5], np.float32), 10.0),
                     (rng.permutation(W.tau_linspace(-1, 2, 777)), 30.0),
                     (W.tau_linspace(0, 1, 1000), 1e4),
                     (np.array([-1e30, -5, 0.25, 0.25, 7, 1e30], np.float32), 5.0)]:
        gout = rng.standard_normal(tau.size).astype(np.float32)
        banner("soft odd", tau.size, lam)
        bad, worst = soft_close(_soft_gpu(E, g, tau, lam), oracle.ecc_soft(g, tau, lam))
        assert bad.size == 0, worst
        bad, worst = soft_close(_soft_gpu(E, g, tau, lam, gout), oracle.ecc_soft_bwd_tau(g, tau, lam, gout))
        assert bad.size == 0, worst


def test_soft_64cube_all_thresholds(E):
    g, tau, extra = W.make_workload("c5_256cube_soft", shape=(64, 64, 64))
    banner("soft 64^3")
    bad, worst = soft_close(_soft_gpu(E, g, tau, extra["lam"]), oracle.ecc_soft(g, tau, extra["lam"]))
    assert bad.size == 0, worst
    gout = extra["grad_out"]
    bad, worst = soft_close(_soft_gpu(E, g, tau, extra["lam"], gout),
                            oracle.ecc_soft_bwd_tau(g, tau, extra["lam"], gout))
    assert bad.size == 0, worst


@pytest.mark.timeout(300)
def test_config_256cube_soft(E):
    """All 256 forward and dL/dtau outputs against the oracle's stored curves;
    the stored backward is for an upstream gradient of ones, and the
    threshold Jacobian is diagonal, so output k scales by g_k."""
    g, tau, extra = W.make_workload("c5_256cube_soft")
    lam, gout = extra["lam"], extra["grad_out"]
    rec = golden_curves.load("c5_256cube_soft")
    assert golden_curves.same_inputs(rec, g, tau) and rec["lam"] == lam
    banner("soft c5 fwd")
    f = _soft_gpu(E, g, tau, lam)
    bad, worst = soft_close(f, np.array(rec["soft"]))
    assert bad.size == 0, (bad[:5], worst)
    banner("soft c5 bwd")
    b = _soft_gpu(E, g, tau, lam, gout)
    bad, worst = soft_close(b, gout.astype(np.float64) * np.array(rec["soft_bwd_unit"]))
    assert bad.size == 0, (bad[:5], worst)


def test_soft_large_lambda_matches_hard_gpu(E):
    rng = np.random.default_rng(29)
    g = (rng.integers(0, 20, (30, 31, 32)) / 20).astype(np.float32)
    tau = (np.arange(-1, 21) / 20 + 0.01).astype(np.float32)
    banner("soft lambda->inf")
    s = _soft_gpu(E, g, tau, 1e6)
    h = _hard_gpu(E, g, tau)
    assert np.max(np.abs(s - h)) < 1e-3


def test_autograd_layer(E):
    import torch
    rng = np.random.default_rng(31)
    g = _dev(rng.random((20, 21, 22), dtype=np.float32))
    tau = torch.tensor(W.tau_linspace(0, 1, 64)).cuda().requires_grad_(True)
    banner("autograd")
    s = E.soft_ecc(g, tau, 25.0)
    (s * torch.arange(64, device=s.device)).sum().backward()
    want = oracle.ecc_soft_bwd_tau(g.cpu().numpy(), tau.detach().cpu().numpy(), 25.0,
                                   np.arange(64, dtype=np.float32))
    bad, worst = soft_close(tau.grad.cpu().numpy(), want)
    assert bad.size == 0, worst


# ------------------------------------------------------------------ errors
def test_errors_raise(E):
    import torch
    g = torch.zeros((4, 4), device="cuda")
    tau = torch.zeros(4, device="cuda")
    small = torch.zeros(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(E.EccError) as ei:
        E.ecc_hard_2d(g, tau, ws=small)
    assert ei.value.status == 6
    with pytest.raises(E.EccError) as ei:
        E.ecc_soft_fwd(g, tau, -1.0)
    assert ei.value.status == 5
    with pytest.raises(E.EccError) as ei:
        E.ecc_hard_2d(g, torch.zeros(9000, device="cuda"))
    assert ei.value.status == 4
    with pytest.raises(TypeError):
        E.ecc_hard_2d(g.double(), tau)
    # the failed calls enqueued nothing: a normal call still works
    assert E.ecc_hard_2d(g, tau).cpu().tolist() == [1, 1, 1, 1]
