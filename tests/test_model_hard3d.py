"""The lane-level model of the float 3D hard tile (tests/model_hard3d.py)
against the oracle, on the CPU: full, partial and element-load chunks, the
three binning modes, tile heights of 1, 2 and 4 rows, and the 5 x 300 x 257
grid with duplicated thresholds (unaligned rows, per-bucket scan)."""

import zlib

import numpy as np
import pytest

import oracle
from euler_characteristic_curves_amd import workloads as W
from tests import model_hard3d as M


def _case(shape, kind, H):
    rng = np.random.default_rng(zlib.crc32(repr((shape, kind, H)).encode()))
    g = rng.random(shape, dtype=np.float32)
    if kind == "lin":
        tau = W.tau_linspace(float(g.min()), float(g.max()), H)
    elif kind == "dups":
        tau = np.sort(rng.choice(np.unique(g), size=H)).astype(np.float32)
    else:
        tau = rng.uniform(-0.2, 1.2, H).astype(np.float32)
    return g, tau


@pytest.mark.parametrize("shape,kind,H,TY,want_kind", [
    ((4, 9, 300), "lin", 97, 4, "lut1"),        # aligned rows: a full and a partial chunk
    ((3, 7, 260), "dups", 64, 4, "lut2"),
    ((3, 6, 36), "lin", 33, 2, "lut1"),         # one partial chunk
    ((4, 6, 300), "unsorted", 50, 2, "search"),
    ((3, 7, 259), "lin", 64, 1, "lut1"),        # unaligned rows: element loads
    ((2, 5, 257), "dups", 40, 2, "lut2"),
])
def test_model_matches_oracle(shape, kind, H, TY, want_kind):
    g, tau = _case(shape, kind, H)
    got, k = M.emulate(g, tau, TY=TY, TZ=2, loads="partial")
    assert k == want_kind
    assert np.array_equal(got, oracle.ecc_hard(g, tau))


def test_model_with_the_kernels_tile_heights():
    """As the kernel routes them: full chunks of aligned rows in 4-row tiles,
    the partial chunk of each row in 2-row tiles (rows 300 and 600 long)."""
    for shape in ((3, 9, 300), (2, 7, 600)):
        g, tau = _case(shape, "lin", 128)
        got, k = M.emulate(g, tau, TY=4, TZ=2, loads="partial", partial_ty=2)
        assert k == "lut1"
        assert np.array_equal(got, oracle.ecc_hard(g, tau))


@pytest.mark.parametrize("offset,width,want_kind", [
    (1e6, 1.0, "lut1"),       # large map offset next to a range of 16 ulps
    (-3e7, 64.0, "lut2"),     # the biased addend's rounding puts two thresholds in a bucket
    (1.0, 1e-6, "lut1"),      # a range of a few ulps
])
def test_model_bucket_map_far_from_zero(offset, width, want_kind):
    """Grids in a narrow band far from zero, with every distinct value as a
    threshold: the 2^23-biased bucket map still bins exactly."""
    rng = np.random.default_rng(zlib.crc32(repr((offset, width)).encode()))
    g = (offset + width * rng.random((3, 9, 300))).astype(np.float32)
    tau = np.unique(g).astype(np.float32)
    got, k = M.emulate(g, tau, TY=4, TZ=2, loads="partial", partial_ty=2)
    assert k == want_kind
    assert np.array_equal(got, oracle.ecc_hard(g, tau))


def test_model_on_the_unaligned_duplicated_threshold_grid():
    """5 x 300 x 257 float32 with 256 duplicated thresholds, drawn as the GPU
    random-shape parity test draws them: the element-load tile with the
    per-bucket scan reproduces the oracle exactly."""
    shape = (5, 300, 257)
    rng = np.random.default_rng(zlib.crc32(repr((shape, "f32")).encode()))
    g = rng.random(shape, dtype=np.float32)
    tau = np.sort(rng.choice(np.unique(g.astype(np.float32)), size=256)).astype(np.float32)
    got, k = M.emulate(g, tau, TZ=2)
    assert k == "lut2"
    assert np.array_equal(got, oracle.ecc_hard(g, tau))


def test_model_detects_a_swapped_edge():
    """The model is sensitive to its edge handling: a copy of it with the left
    and right neighbours of the third sequence swapped no longer matches."""
    import inspect
    import types
    src = inspect.getsource(M)
    planted = src.replace("tele(s3, l3, r3, -1)", "tele(s3, r3, l3, -1)")
    assert planted != src
    bad = types.ModuleType("model_hard3d_planted")
    exec(compile(planted, "model_hard3d_planted", "exec"), bad.__dict__)
    g, tau = _case((3, 7, 260), "lin", 64)
    got, _ = bad.emulate(g, tau, TY=4, TZ=2, loads="partial")
    assert not np.array_equal(got, oracle.ecc_hard(g, tau))
