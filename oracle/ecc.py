"""Plain numpy reference for hard and soft Euler characteristic curves.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the product.

Source: page "Scalable GPU-Accelerated Euler Characteristic Curves:
Optimization and Differentiable Learning for PyTorch" (paper notes), sections
"Method / Key designs" (full-sweep kernel; differentiable ECC layer; local
Euler-coefficient computation).

The complex (a reading, the page does not name it): a 2D or 3D grid is the
vertex set of a cubical complex (V-construction).  Cells are vertices, the
edges between axis-adjacent voxels, the axis-aligned 2x2 squares and (3D) the
2x2x2 cubes.  A cell's filtration value is the maximum of its corner values,
its sign is (-1)^dim.  The sublevel complex at tau holds the cells whose value
is <= tau (the page's hard indicator of X(p) <= tau).

Precision: comparisons are exact (values and thresholds widened to float64,
which is exact for float32 and uint8); soft quantities are float64.
"""

import itertools

import numpy as np

__all__ = [
    "cell_values", "cell_counts", "first_k_bins", "ecc_hard", "ecc_at",
    "sigmoid", "ecc_soft", "ecc_soft_percell", "ecc_soft_at",
    "ecc_soft_bwd_tau", "ecc_soft_bwd_at", "ecc_at_many", "ecc_soft_at_many",
    "ecc_soft_bwd_at_many", "ecc_soft_bwd_grid", "ecc_soft_bwd_grid_at", "ecc_hard_batched",
    "height_values", "height_bwd",
]


def _check_grid(grid):
    grid = np.asarray(grid)
    if grid.ndim not in (2, 3):
        raise ValueError("grid must be 2D or 3D")
    if grid.size == 0:
        raise ValueError("grid must be non-empty")
    return grid


def cell_values(grid):
    """Yield (values, dim) for every cell type of the V-construction complex.

    A cell type is an extent e in {0,1}^d; the cell anchored at voxel p has
    corners p + o for every o <= e (componentwise).  Its value is the max of
    its corners and its dimension is sum(e).  Only cells whose corners all lie
    inside the grid exist.  ``values`` holds one entry per anchor p.
    (Key designs: each voxel owns its vertex and its +x/+y(/+z) edges,
    squares and cube; a cell's value is the max of its corners.)
    """
    grid = _check_grid(grid)
    shape = grid.shape
    for ext in itertools.product((0, 1), repeat=grid.ndim):
        anchors = [n - e for n, e in zip(shape, ext)]
        if min(anchors) <= 0:
            continue
        val = None
        for off in itertools.product(*[range(e + 1) for e in ext]):
            corner = grid[tuple(slice(o, o + a) for o, a in zip(off, anchors))]
            val = corner.copy() if val is None else np.maximum(val, corner)
        yield val, sum(ext)


def cell_counts(shape):
    """Number of cells of each dimension in the full box complex of ``shape``."""
    counts = [0] * (len(shape) + 1)
    for ext in itertools.product((0, 1), repeat=len(shape)):
        n = 1
        for s, e in zip(shape, ext):
            n *= max(s - e, 0)
        counts[sum(ext)] += n
    return counts


def _tau64(tau):
    tau = np.asarray(tau)
    if tau.ndim != 1 or tau.size == 0:
        raise ValueError("tau must be a non-empty 1-D array")
    return tau.astype(np.float32).astype(np.float64)


def first_k_bins(values, tau):
    """bin(v) = min{k : v <= tau_k}, or H when no threshold reaches v.

    Reading of the page (it only says each block keeps an H-bin histogram):
    a cell is counted from the first threshold that admits it, with an exact
    float comparison and no tolerance.  For non-decreasing tau this is
    numpy's left-sided searchsorted; for any other order the definition is
    evaluated literally (chunked v <= tau_k table and first true index).
    """
    t = _tau64(tau)
    v = np.asarray(values).astype(np.float64).ravel()
    H = t.size
    if np.all(t[1:] >= t[:-1]):
        return np.searchsorted(t, v, side="left").astype(np.int64)
    out = np.empty(v.size, dtype=np.int64)
    step = max(1, (1 << 22) // H)
    for i in range(0, v.size, step):
        le = v[i:i + step, None] <= t[None, :]
        hit = le.any(axis=1)
        out[i:i + step] = np.where(hit, le.argmax(axis=1), H)
    return out


def _z_slabs(grid, slab):
    """Split a 3D grid into z-slabs [z0, z1) with a one-plane halo on top.

    Cells anchored in [z0, z1) are exactly the cells of grid[z0:z1+1] whose
    anchor plane is < z1 - z0, so every cell of the whole grid is produced
    once.  2D grids are a single slab.
    """
    if grid.ndim == 2 or slab is None or grid.shape[0] <= slab:
        yield grid, None
        return
    nz = grid.shape[0]
    for z0 in range(0, nz, slab):
        z1 = min(z0 + slab, nz)
        yield grid[z0:min(z1 + 1, nz)], z1 - z0


def _slab_cells(sub, keep):
    for val, dim in cell_values(sub):
        if keep is not None:
            val = val[:keep]
        yield val, dim


def ecc_hard(grid, tau, slab=32):
    """Hard ECC: out[k] = sum over cells c of (-1)^dim(c) * [bin(c) <= k].

    Steps as on the page: every cell contributes its sign to the histogram
    bin of its first admitting threshold (per-block H-bin histogram), and the
    curve is the running sum of that histogram.  For non-decreasing tau,
    out[k] is the Euler characteristic of the sublevel complex at tau_k.
    Returns int64[H].  3D grids are processed in z-slabs to bound memory.
    """
    grid = _check_grid(grid)
    t = _tau64(tau)
    H = t.size
    hist = np.zeros(H + 1, dtype=np.int64)
    for sub, keep in _z_slabs(grid, slab):
        for val, dim in _slab_cells(sub, keep):
            b = first_k_bins(val, t)
            hist += (-1) ** dim * np.bincount(b, minlength=H + 1).astype(np.int64)
    return np.cumsum(hist[:H]).astype(np.int64)


def ecc_at(grid, t, slab=32):
    """Euler characteristic of the sublevel complex {c : value(c) <= t}.

    The plain definition chi = #V - #E + #F (- #C) at one threshold, counted
    directly (no binning).  Used to check single outputs of large grids.
    """
    grid = _check_grid(grid)
    t = float(np.float32(t))
    chi = 0
    for sub, keep in _z_slabs(grid, slab):
        for val, dim in _slab_cells(sub, keep):
            chi += (-1) ** dim * int(np.count_nonzero(val.astype(np.float64) <= t))
    return chi


def ecc_at_many(grid, ts, slab=32):
    """ecc_at for several thresholds with one pass over the cells (int64 array)."""
    grid = _check_grid(grid)
    t = np.asarray(ts, dtype=np.float32).astype(np.float64).ravel()
    chi = np.zeros(t.size, dtype=np.int64)
    for sub, keep in _z_slabs(grid, slab):
        for val, dim in _slab_cells(sub, keep):
            v = val.astype(np.float64)
            for i, ti in enumerate(t):
                chi[i] += (-1) ** dim * int(np.count_nonzero(v <= ti))
    return chi


def sigmoid(x):
    """Logistic function 1/(1+exp(-x)) in float64, evaluated via exp(-|x|)."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def _dsig(x):
    """sigma(x) * sigma(-x) = e/(1+e)^2 with e = exp(-|x|) (even in x)."""
    e = np.exp(-np.abs(np.asarray(x, dtype=np.float64)))
    return e / (1.0 + e) ** 2


def _check_lambda(lam):
    lam = float(np.float32(lam))
    if not np.isfinite(lam) or lam <= 0:
        raise ValueError("lambda must be finite and > 0")
    return lam


def _grouped_weights(grid, slab=32):
    """Distinct cell values and the sum of the signs of the cells holding each.

    sum_c sign_c f(v_c) = sum_u (sum_{c: v_c = u} sign_c) f(u): an exact
    regrouping that keeps the sigmoid sweep below size #distinct values.
    """
    vals, wts = [], []
    for sub, keep in _z_slabs(_check_grid(grid), slab):
        for val, dim in _slab_cells(sub, keep):
            u, cnt = np.unique(val.astype(np.float64).ravel(), return_counts=True)
            vals.append(u)
            wts.append((-1) ** dim * cnt.astype(np.int64))
    v = np.concatenate(vals)
    w = np.concatenate(wts)
    u, inv = np.unique(v, return_inverse=True)
    wsum = np.zeros(u.size, dtype=np.int64)
    np.add.at(wsum, inv, w)
    nz = wsum != 0
    return u[nz], wsum[nz]


def _sweep(u, w, t, lam, fn, chunk=1 << 16):
    out = np.zeros(t.size, dtype=np.float64)
    wf = w.astype(np.float64)
    for i in range(0, u.size, chunk):
        x = lam * (t[None, :] - u[i:i + chunk, None])
        out += wf[i:i + chunk] @ fn(x)
    return out


def ecc_soft(grid, tau, lam, slab=32):
    """Soft ECC: S_k = sum_c (-1)^dim(c) * sigmoid(lam * (tau_k - value(c))).

    Differentiable ECC layer: the sublevel indicator of value <= tau is
    replaced by sigma_lambda(tau - value) with sigma_lambda(z) = 1/(1+exp(-lam
    z)) (reading: lambda is an inverse temperature), applied per cell with the
    cell value defined as for the hard curve.  lambda -> infinity gives back
    the hard curve.  float64 throughout; cells are grouped by exact value.
    """
    t = _tau64(tau)
    lam = _check_lambda(lam)
    u, w = _grouped_weights(grid, slab)
    return _sweep(u, w, t, lam, sigmoid)


def ecc_soft_percell(grid, tau, lam):
    """Same as ecc_soft without the grouping: one sigmoid per cell (small grids)."""
    t = _tau64(tau)
    lam = _check_lambda(lam)
    out = np.zeros(t.size, dtype=np.float64)
    for val, dim in cell_values(grid):
        v = val.astype(np.float64).ravel()
        out += (-1) ** dim * sigmoid(lam * (t[None, :] - v[:, None])).sum(axis=0)
    return out


def ecc_soft_at(grid, t, lam, slab=32):
    """One soft-ECC output: sum_c sign_c sigmoid(lam (t - value(c))), per cell."""
    t = float(np.float32(t))
    lam = _check_lambda(lam)
    acc = 0.0
    for sub, keep in _z_slabs(_check_grid(grid), slab):
        for val, dim in _slab_cells(sub, keep):
            acc += (-1) ** dim * float(sigmoid(lam * (t - val.astype(np.float64))).sum())
    return acc


def ecc_soft_at_many(grid, ts, lam, slab=32):
    """ecc_soft_at for several thresholds with one pass over the cells (float64 array)."""
    t = np.asarray(ts, dtype=np.float32).astype(np.float64).ravel()
    lam = _check_lambda(lam)
    acc = np.zeros(t.size, dtype=np.float64)
    for sub, keep in _z_slabs(_check_grid(grid), slab):
        for val, dim in _slab_cells(sub, keep):
            v = val.astype(np.float64)
            for i, ti in enumerate(t):
                acc[i] += (-1) ** dim * float(sigmoid(lam * (ti - v)).sum())
    return acc


def ecc_soft_bwd_at_many(grid, ts, lam, gs, slab=32):
    """ecc_soft_bwd_at for several thresholds with one pass over the cells."""
    t = np.asarray(ts, dtype=np.float32).astype(np.float64).ravel()
    g = np.asarray(gs, dtype=np.float32).astype(np.float64).ravel()
    lam = _check_lambda(lam)
    acc = np.zeros(t.size, dtype=np.float64)
    for sub, keep in _z_slabs(_check_grid(grid), slab):
        for val, dim in _slab_cells(sub, keep):
            v = val.astype(np.float64)
            for i, ti in enumerate(t):
                acc[i] += (-1) ** dim * float(_dsig(lam * (ti - v)).sum())
    return g * lam * acc


def ecc_soft_bwd_tau(grid, tau, lam, grad_out, slab=32):
    """dL/dtau_k = g_k * lam * sum_c (-1)^dim(c) sigma(x) sigma(-x), x = lam(tau_k - v_c).

    The analytic backward of ecc_soft with respect to the thresholds.  Each
    S_k depends on tau_k alone, so the Jacobian is diagonal and the upstream
    gradient g_k scales output k.  float64; cells grouped by exact value.
    """
    t = _tau64(tau)
    lam = _check_lambda(lam)
    g = np.asarray(grad_out).astype(np.float32).astype(np.float64)
    if g.shape != t.shape:
        raise ValueError("grad_out must have the shape of tau")
    u, w = _grouped_weights(grid, slab)
    return g * lam * _sweep(u, w, t, lam, _dsig)


def ecc_soft_bwd_at(grid, t, lam, g, slab=32):
    """One output of ecc_soft_bwd_tau, summed per cell without grouping."""
    t = float(np.float32(t))
    lam = _check_lambda(lam)
    g = float(np.float32(g))
    acc = 0.0
    for sub, keep in _z_slabs(_check_grid(grid), slab):
        for val, dim in _slab_cells(sub, keep):
            acc += (-1) ** dim * float(_dsig(lam * (t - val.astype(np.float64))).sum())
    return g * lam * acc


# ------------------------------------------------------------ grid gradient
# The differentiable ECC layer of the page ("Method / Key designs") has an
# analytic backward; the gradient with respect to the grid values follows from
# the same definition.  A cell's value is the max of its corners, so d v_c /
# d X(p) is 1 for the corner holding the max and 0 for the others.  Ties (a
# reading; the page does not discuss them): the max goes to the first corner
# in index order (C order, x fastest) among those holding it, so the gradient
# is one subgradient of the max, the one a first-index argmax picks.

def _h_of(u, t, lam, g, chunk=1 << 15):
    """h(u) = sum_k g_k sigma(x) sigma(-x), x = lam (tau_k - u), for each u (float64)."""
    out = np.empty(u.size, dtype=np.float64)
    for i in range(0, u.size, chunk):
        x = lam * (t[None, :] - u[i:i + chunk, None])
        out[i:i + chunk] = _dsig(x) @ g
    return out


def _grad_inputs(grid, tau, lam, grad_out):
    grid = _check_grid(grid)
    t = _tau64(tau)
    lam = _check_lambda(lam)
    g = np.asarray(grad_out).astype(np.float32).astype(np.float64)
    if g.shape != t.shape:
        raise ValueError("grad_out must have the shape of tau")
    return grid, t, lam, g


def ecc_soft_bwd_grid(grid, tau, lam, grad_out):
    """dL/dX(p) for L = sum_k g_k S_k, S = ecc_soft(grid, tau, lam).

    d S_k / d v_c = -lam sigma(x) sigma(-x) with x = lam (tau_k - v_c), and
    d v_c / d X(p) = [p is the argmax corner of c]; so every cell passes
    -lam (-1)^dim(c) h(v_c) to its argmax corner, h(v) = sum_k g_k sigma sigma'.
    Written as that scatter, cell type by cell type (float64).
    """
    grid, t, lam, g = _grad_inputs(grid, tau, lam, grad_out)
    X = grid.astype(np.float64)
    shape = X.shape
    index = np.arange(X.size, dtype=np.int64).reshape(shape)
    out = np.zeros(X.size, dtype=np.float64)
    for ext in itertools.product((0, 1), repeat=X.ndim):
        anchors = [n - e for n, e in zip(shape, ext)]
        if min(anchors) <= 0:
            continue
        offs = list(itertools.product(*[range(e + 1) for e in ext]))  # increasing index order
        vals = np.stack([X[tuple(slice(o, o + a) for o, a in zip(off, anchors))] for off in offs])
        idxs = np.stack([index[tuple(slice(o, o + a) for o, a in zip(off, anchors))] for off in offs])
        am = np.argmax(vals, axis=0)  # first corner holding the max
        v = np.take_along_axis(vals, am[None], 0)[0].ravel()
        tgt = np.take_along_axis(idxs, am[None], 0)[0].ravel()
        u, inv = np.unique(v, return_inverse=True)
        contrib = -lam * (-1) ** sum(ext) * _h_of(u, t, lam, g)[inv]
        np.add.at(out, tgt, contrib)
    return out.reshape(shape)


def ecc_soft_bwd_grid_at(grid, points, tau, lam, grad_out):
    """ecc_soft_bwd_grid at selected voxels (a list of index tuples), float64.

    Per voxel p: every cell holding p whose max goes to p has value X(p), so
    dL/dX(p) = -lam c(p) h(X(p)) with c(p) the signed count of those cells.
    The cells are enumerated one by one around p (for large grids, where the
    full scatter does not fit).
    """
    grid, t, lam, g = _grad_inputs(grid, tau, lam, grad_out)
    X = grid.astype(np.float64)
    shape = X.shape
    res = []
    for p in points:
        p = tuple(int(c) for c in p)
        c = 0
        for ext in itertools.product((0, 1), repeat=X.ndim):
            for o in itertools.product(*[range(e + 1) for e in ext]):
                a = tuple(pi - oi for pi, oi in zip(p, o))
                if any(ai < 0 or ai + e >= n for ai, e, n in zip(a, ext, shape)):
                    continue  # cell sticks out of the grid
                corners = [tuple(ai + qi for ai, qi in zip(a, q))
                           for q in itertools.product(*[range(e + 1) for e in ext])]
                best = max(corners, key=lambda q: (X[q], -np.ravel_multi_index(q, shape)))
                if best == p:
                    c += (-1) ** sum(ext)
        h = float(_h_of(np.array([X[p]]), t, lam, g)[0]) if c else 0.0
        res.append(-lam * c * h)
    return np.array(res, dtype=np.float64)


# ------------------------------------------------------------------ batches
def ecc_hard_batched(grids, tau):
    """Hard ECC of each grid of a batch: int64[B, H].

    A batch is a set of independent grids (the page lists batched execution
    among its next steps, section "Limitations and outlook"); no cell joins two
    grids.  ``tau`` is one threshold array for all grids ([H]) or one row per
    grid ([B, H]).  Written as the loop it is.
    """
    grids = np.asarray(grids)
    tau = np.asarray(tau)
    if grids.ndim not in (3, 4):
        raise ValueError("grids must be [B, ny, nx] or [B, nz, ny, nx]")
    rows = [ecc_hard(grids[b], tau if tau.ndim == 1 else tau[b]) for b in range(grids.shape[0])]
    return np.stack(rows)


# ------------------------------------------------------- directional heights
# The page's single-direction layer adds a learnable direction u and scale
# alpha, with gradients through both, and names the multi-direction transform
# as the complete version (sections "Method / Key designs / differentiable ECC
# layer" and "Limitations and outlook").  It does not define the height
# function on a grid; the reading taken here is
#     f_d(p) = X(p) + alpha_d * <u_d, p>,
# with p the integer voxel index (slowest axis first).  A voxel at +inf never
# enters, so X = 0 on a shape and +inf off it gives the shape's directional
# filtration, and a plain intensity grid gets a tilted one.  The curves of
# direction d are those of the grid f_d.

def height_values(grid, dirs, alpha):
    """f[d] = grid + alpha[d] * <dirs[d], p> in float32, float32[D, *shape].

    The arithmetic is fixed so that it can be reproduced bit for bit: each
    product and sum rounded to float32 in the order
        h = (u_0 p_0 + u_1 p_1) [+ u_2 p_2],   f = X + alpha * h,
    with no fused multiply-add.
    """
    X = np.asarray(grid, dtype=np.float32)
    if X.ndim not in (2, 3):
        raise ValueError("grid must be 2D or 3D")
    U = np.asarray(dirs, dtype=np.float32).reshape(-1, X.ndim)
    A = np.asarray(alpha, dtype=np.float32).reshape(-1)
    if A.size != U.shape[0]:
        raise ValueError("one alpha per direction")
    idx = [np.arange(n, dtype=np.float32).reshape([-1 if a == i else 1 for a in range(X.ndim)])
           for i, n in enumerate(X.shape)]
    out = np.empty((U.shape[0],) + X.shape, dtype=np.float32)
    for d in range(U.shape[0]):
        h = np.float32(U[d, 0]) * idx[0]
        for i in range(1, X.ndim):
            h = h + np.float32(U[d, i]) * idx[i]
        out[d] = X + np.float32(A[d]) * h
    return out


def height_bwd(grad_h, dirs, alpha):
    """Chain rule of height_values, float64.

    Given G[d] = dL/df[d]: dL/dX = sum_d G[d]; with M[d, i] = sum_p G[d](p) p_i,
    dL/du[d, i] = alpha[d] M[d, i] and dL/dalpha[d] = sum_i u[d, i] M[d, i].
    """
    G = np.asarray(grad_h, dtype=np.float64)
    nd = G.ndim - 1
    U = np.asarray(dirs, dtype=np.float32).astype(np.float64).reshape(-1, nd)
    A = np.asarray(alpha, dtype=np.float32).astype(np.float64).reshape(-1)
    M = np.zeros((G.shape[0], nd))
    for i, n in enumerate(G.shape[1:]):
        coord = np.arange(n, dtype=np.float64).reshape([-1 if a == i else 1 for a in range(nd)])
        M[:, i] = (G * coord).reshape(G.shape[0], -1).sum(axis=1)
    return G.sum(axis=0), A[:, None] * M, (U * M).sum(axis=1)
