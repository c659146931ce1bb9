"""Error bounds that the soft ECC entry points document for themselves (test
infrastructure).  They are computed from the oracle's merged cell terms; the
tests compare the GPU results with the oracle against these bounds.

For a threshold tau_k and a cell value v, x = lambda (tau_k - v).  One float32
sigmoid carries a relative error of at most (6 + 1.5 |x|) 2^-24 in the forward
and (8 + 1.5 |x|) 2^-24 for s(1 - s) in the threshold backward; the workgroup
sums are combined in fixed point with resolution 2^-s, W workgroups each
rounding once; the float32 output rounds once more.
"""
import math

import numpy as np

from oracle import ecc as OE

TILE_VOXELS = 512


def fixed_point(nvox):
    """(W, s): workgroups on one grid (at most one per 512-voxel tile) and the
    number of fraction bits of the fixed-point combination."""
    bits = 0
    while bits < 62 and (1 << bits) < 8 * nvox + 8:
        bits += 1
    return math.ceil(nvox / TILE_VOXELS), 61 - bits


def _sig(x):
    return np.where(x >= 0, 1.0 / (1.0 + np.exp(-np.abs(x))), np.exp(-np.abs(x)) / (1.0 + np.exp(-np.abs(x))))


def soft_bounds(grid, tau, lam, grad_out=None):
    """Documented error bounds: (forward[H], threshold backward[H]) before the
    output rounding; the backward's is None without grad_out."""
    u, w = OE._grouped_weights(grid)
    aw = np.abs(w).astype(np.float64)
    t = np.asarray(tau, np.float32).astype(np.float64)
    W, s = fixed_point(int(np.prod(grid.shape)))
    quant = 0.5 * W * 2.0 ** -s
    fwd = np.empty(t.size)
    bwd = np.empty(t.size)
    for k in range(t.size):
        x = lam * (t[k] - u)
        sg = _sig(x)
        fwd[k] = float(aw @ ((6.0 + 1.5 * np.abs(x)) * 2.0 ** -24 * sg)) + quant
        ds = sg * _sig(-x)
        bwd[k] = float(aw @ ((8.0 + 1.5 * np.abs(x)) * 2.0 ** -24 * ds)) + quant
    if grad_out is None:
        return fwd, None
    g = np.abs(np.asarray(grad_out, np.float32).astype(np.float64))
    return fwd, lam * g * bwd


def within(got, want, bound):
    """Indices where |got - want| exceeds bound plus the output rounding."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    lim = bound + 2.0 ** -24 * np.maximum(np.abs(got), np.abs(want))
    return np.nonzero(~(np.abs(got - want) <= lim))[0]
