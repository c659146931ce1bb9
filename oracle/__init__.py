"""CPU oracle for Euler characteristic curves of dense 2D/3D grids.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, obviously correct
reference that the HIP library is checked against.  Only the test suite, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import it.  The product path (``euler_characteristic_curves_amd``) never
imports, links or calls anything in here, and nothing in here imports the
product path: the two share no code.

Everything follows the page "Scalable GPU-Accelerated Euler Characteristic
Curves: Optimization and Differentiable Learning for PyTorch" (NeurIPS 2025
NeurReps workshop paper notes), sections "Method / Key designs": the
full-sweep kernel (per-block histogram of H bins turned into a curve), the
differentiable ECC layer (sigmoid relaxation of the sublevel indicator) and
the local Euler-coefficient decomposition.  Readings of points the page leaves
open are listed in each function's docstring.

Pinning status (what checks this oracle against something other than itself):
  * ecc_hard / ecc_at      -- pinned: brute-force V-E+F(-C) cell counting,
                               2D union-find beta0-beta1, scipy.ndimage.label,
                               closed forms, invariants, metamorphic checks,
                               hand-derived golden fixtures.
  * ecc_soft / ecc_soft_at -- pinned: per-cell math.exp brute force, constant
                               grid closed form, lambda -> infinity limit.
  * ecc_soft_bwd_tau       -- pinned: central finite differences of the
                               forward, integral identity (sum of signs = 1).
  * ecc_soft_bwd_grid(_at) -- pinned: central finite differences of a
                               per-cell brute-force forward with respect to
                               each voxel on tie-free grids, the sum rule
                               (translating the grid by s moves every cell
                               value by s), per-voxel vs scatter agreement.
  * height_values / height_bwd -- pinned: hand-computed heights, the
                               directional curve of a box (a step) and of a
                               frame (0, 1, 0) by brute force, central finite
                               differences of the whole soft pipeline in u,
                               alpha and the grid.
  * at the 256^3 soft size: the forward and the threshold backward of a
    256^3 checkerboard against their two-term closed form (every edge,
    square and cube takes the high value, the box has chi = 1).
"""

from .ecc import (  # noqa: F401
    cell_values,
    cell_counts,
    first_k_bins,
    ecc_hard,
    ecc_hard_batched,
    height_values,
    height_bwd,
    ecc_at,
    ecc_at_many,
    ecc_soft,
    ecc_soft_percell,
    ecc_soft_at,
    ecc_soft_at_many,
    ecc_soft_bwd_tau,
    ecc_soft_bwd_at,
    ecc_soft_bwd_at_many,
    ecc_soft_bwd_grid,
    ecc_soft_bwd_grid_at,
    sigmoid,
)
