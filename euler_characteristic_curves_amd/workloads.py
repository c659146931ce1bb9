"""Seeded synthetic inputs for the hard and soft ECC workloads.

This module only draws random grids and builds threshold / upstream-gradient
arrays.  It holds none of the Euler-characteristic arithmetic, so both the
HIP path (tests, bench) and the CPU oracle can take their inputs from here.

The page ("Scalable GPU-Accelerated Euler Characteristic Curves", section
"Key experimental data") times unnamed synthetic 2D grids of 128^2..8192^2 and
3D grids of 128^3..1024^3 and states no seed, dtype, threshold count or value
distribution.  The recipes below stand in for those grids:

  * iid uniform float32 in [0, 1)            numpy default_rng(seed).random
  * iid uniform uint8 in {0..255}            numpy default_rng(seed).integers
  * Gaussian random field: iid N(0,1) float64 white noise smoothed by a
    periodic Gaussian filter (FFT multiply by exp(-2 pi^2 s^2 |nu|^2), nu in
    cycles per voxel), cast to float32.
  * thresholds: k/255, the integers k, or linspace(min, max, H) computed in
    float64, cast to float32, with the end points pinned to the exact grid
    min and max so the last threshold admits every cell.
"""

import numpy as np

__all__ = [
    "uniform_f32", "uniform_u8", "gaussian_random_field",
    "tau_k_over", "tau_integers", "tau_linspace", "upstream_grad",
    "WORKLOADS", "make_workload",
]


def uniform_f32(shape, seed):
    """iid uniform [0, 1) float32 (numpy's float32 generator, 2^-24 steps)."""
    return np.random.default_rng(seed).random(shape, dtype=np.float32)


def uniform_u8(shape, seed):
    """iid uniform {0..255} uint8."""
    return np.random.default_rng(seed).integers(0, 256, size=shape, dtype=np.uint8)


def gaussian_random_field(shape, sigma, seed):
    """Periodic Gaussian-smoothed white noise, float32.

    White noise N(0,1) in float64 is multiplied in Fourier space by the
    transfer function of a Gaussian of standard deviation ``sigma`` voxels
    (periodic boundary), then cast to float32.  No normalisation is applied.
    """
    from scipy import fft as sfft
    rng = np.random.default_rng(seed)
    white = rng.standard_normal(shape)
    spec = sfft.rfftn(white, workers=-1)
    del white
    filt = None
    for ax, n in enumerate(shape):
        nu = sfft.rfftfreq(n) if ax == len(shape) - 1 else sfft.fftfreq(n)
        g = np.exp(-2.0 * np.pi ** 2 * sigma ** 2 * nu ** 2)
        bshape = [1] * len(shape)
        bshape[ax] = g.size
        g = g.reshape(bshape)
        filt = g if filt is None else filt * g
    spec *= filt
    out = sfft.irfftn(spec, s=shape, workers=-1)
    return out.astype(np.float32)


def tau_k_over(H, denom):
    """tau_k = float32(k / denom), k = 0..H-1."""
    return (np.arange(H, dtype=np.float64) / denom).astype(np.float32)


def tau_integers(H):
    """tau_k = float32(k), k = 0..H-1."""
    return np.arange(H, dtype=np.float32)


def tau_linspace(lo, hi, H):
    """linspace(lo, hi, H) in float64 cast to float32, ends pinned to lo/hi."""
    lo32, hi32 = np.float32(lo), np.float32(hi)
    t = np.linspace(float(lo32), float(hi32), H).astype(np.float32)
    t[0] = lo32
    t[-1] = hi32
    return t


def upstream_grad(H, seed):
    """Upstream gradient g_k ~ N(0, 1), float32."""
    return np.random.default_rng(seed).standard_normal(H).astype(np.float32)


# The five workloads: name -> recipe.  "kind" is hard2d / hard3d / soft3d.
WORKLOADS = {
    "c1_128sq_f32": dict(kind="hard2d", shape=(128, 128), dtype="f32", gen="uniform", seed=1,
                         H=256, tau="k/255"),
    "c2_1024sq_f32_grf": dict(kind="hard2d", shape=(1024, 1024), dtype="f32", gen="grf", sigma=4.0,
                              seed=2, H=1024, tau="linspace"),
    "c3_8192sq_u8": dict(kind="hard2d", shape=(8192, 8192), dtype="u8", gen="uniform", seed=3,
                         H=256, tau="k"),
    "c4a_512cube_f32_grf": dict(kind="hard3d", shape=(512, 512, 512), dtype="f32", gen="grf",
                                sigma=3.0, seed=4, H=512, tau="linspace"),
    "c4b_1024cube_f32": dict(kind="hard3d", shape=(1024, 1024, 1024), dtype="f32", gen="uniform",
                             seed=41, H=512, tau="linspace"),
    "c5_256cube_soft": dict(kind="soft3d", shape=(256, 256, 256), dtype="f32", gen="uniform", seed=5,
                            H=256, tau="linspace01", lam=50.0, gseed=55),
}


def make_workload(name, shape=None):
    """Return (grid, tau, extra) for a named workload, optionally at another shape.

    ``extra`` carries lambda and the upstream gradient for the soft workload.
    """
    w = WORKLOADS[name]
    shape = tuple(shape) if shape is not None else w["shape"]
    if w["gen"] == "grf":
        grid = gaussian_random_field(shape, w["sigma"], w["seed"])
    elif w["dtype"] == "u8":
        grid = uniform_u8(shape, w["seed"])
    else:
        grid = uniform_f32(shape, w["seed"])
    H = w["H"]
    kind = w["tau"]
    if kind == "k/255":
        tau = tau_k_over(H, 255.0)
    elif kind == "k":
        tau = tau_integers(H)
    elif kind == "linspace":
        tau = tau_linspace(grid.min(), grid.max(), H)
    elif kind == "linspace01":
        tau = tau_linspace(0.0, 1.0, H)
    else:
        raise ValueError(kind)
    extra = {}
    if w["kind"] == "soft3d":
        extra["lam"] = w["lam"]
        extra["grad_out"] = upstream_grad(H, w["gseed"])
    return grid, tau, extra
