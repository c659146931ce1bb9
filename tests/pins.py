"""Independent checkers that pin the oracle to the mathematics.

None of these share code with ``oracle/``: they count cells of the sublevel
complex one by one with explicit loops, compute Betti numbers with a
hand-written union-find, or evaluate closed forms.  They are slow and only
meant for tiny grids.
"""

import math

import numpy as np


# ---------------------------------------------------------------- brute force
def brute_chi_2d(g, t):
    """chi = #V - #E + #F of the V-construction sublevel complex, by hand.

    A cell is in the complex iff every corner voxel has value <= t.
    """
    ny, nx = g.shape
    inn = [[float(g[y, x]) <= t for x in range(nx)] for y in range(ny)]
    V = sum(inn[y][x] for y in range(ny) for x in range(nx))
    E = 0
    for y in range(ny):
        for x in range(nx - 1):
            E += inn[y][x] and inn[y][x + 1]
    for y in range(ny - 1):
        for x in range(nx):
            E += inn[y][x] and inn[y + 1][x]
    F = 0
    for y in range(ny - 1):
        for x in range(nx - 1):
            F += inn[y][x] and inn[y][x + 1] and inn[y + 1][x] and inn[y + 1][x + 1]
    return V - E + F


def brute_chi_3d(g, t):
    """chi = #V - #E + #F - #C of the 3D V-construction sublevel complex, by hand."""
    nz, ny, nx = g.shape
    inn = (np.asarray(g, dtype=np.float64) <= t).tolist()

    def on(z, y, x):
        return inn[z][y][x]

    V = E = F = C = 0
    for z in range(nz):
        for y in range(ny):
            for x in range(nx):
                if not on(z, y, x):
                    continue
                V += 1
                # edges toward +x, +y, +z
                if x + 1 < nx and on(z, y, x + 1):
                    E += 1
                if y + 1 < ny and on(z, y + 1, x):
                    E += 1
                if z + 1 < nz and on(z + 1, y, x):
                    E += 1
                # squares in the xy, xz and yz planes
                if x + 1 < nx and y + 1 < ny and on(z, y, x + 1) and on(z, y + 1, x) and on(z, y + 1, x + 1):
                    F += 1
                if x + 1 < nx and z + 1 < nz and on(z, y, x + 1) and on(z + 1, y, x) and on(z + 1, y, x + 1):
                    F += 1
                if y + 1 < ny and z + 1 < nz and on(z, y + 1, x) and on(z + 1, y, x) and on(z + 1, y + 1, x):
                    F += 1
                if x + 1 < nx and y + 1 < ny and z + 1 < nz:
                    corners = [on(z + a, y + b, x + c) for a in (0, 1) for b in (0, 1) for c in (0, 1)]
                    if all(corners):
                        C += 1
    return V - E + F - C


def brute_chi(g, t):
    return brute_chi_2d(g, t) if g.ndim == 2 else brute_chi_3d(g, t)


# ------------------------------------------------------------ union-find 2D
class _UF:
    def __init__(self, n):
        self.p = list(range(n))

    def find(self, a):
        while self.p[a] != a:
            self.p[a] = self.p[self.p[a]]
            a = self.p[a]
        return a

    def union(self, a, b):
        ra, rb = self.find(a), self.find(b)
        if ra != rb:
            self.p[ra] = rb


def betti_2d(g, t):
    """(beta0, beta1) of the 2D sublevel complex by union-find.

    beta0: components of foreground pixels (value <= t) under 4-adjacency
    (the complex's edges).  beta1: holes, i.e. components of background
    pixels under 8-adjacency (a square missing a corner leaves its interior
    open, joining diagonal background pixels) that do not touch the border.
    """
    ny, nx = g.shape
    fg = [[float(g[y, x]) <= t for x in range(nx)] for y in range(ny)]
    uf = _UF(ny * nx + 1)
    outside = ny * nx
    for y in range(ny):
        for x in range(nx):
            i = y * nx + x
            if fg[y][x]:
                if x + 1 < nx and fg[y][x + 1]:
                    uf.union(i, i + 1)
                if y + 1 < ny and fg[y + 1][x]:
                    uf.union(i, i + nx)
            else:
                if y in (0, ny - 1) or x in (0, nx - 1):
                    uf.union(i, outside)
                for dy in (-1, 0, 1):
                    for dx in (-1, 0, 1):
                        yy, xx = y + dy, x + dx
                        if 0 <= yy < ny and 0 <= xx < nx and not fg[yy][xx]:
                            uf.union(i, yy * nx + xx)
    roots_fg = {uf.find(y * nx + x) for y in range(ny) for x in range(nx) if fg[y][x]}
    roots_bg = {uf.find(y * nx + x) for y in range(ny) for x in range(nx) if not fg[y][x]}
    roots_bg.discard(uf.find(outside))
    return len(roots_fg), len(roots_bg)


def betti_2d_scipy(g, t):
    """(beta0, beta1) via scipy.ndimage.label: a library cross-check."""
    from scipy import ndimage
    fg = np.asarray(g, dtype=np.float64) <= t
    _, b0 = ndimage.label(fg, structure=ndimage.generate_binary_structure(2, 1))
    bg = np.pad(~fg, 1, constant_values=True)
    _, nbg = ndimage.label(bg, structure=ndimage.generate_binary_structure(2, 2))
    return b0, nbg - 1


def betti02_3d_scipy(g, t):
    """(beta0, beta2) of the 3D sublevel complex via scipy.ndimage.label.

    beta0: 6-connected foreground components; beta2: 26-connected background
    components that do not reach the border (enclosed cavities).
    """
    from scipy import ndimage
    fg = np.asarray(g, dtype=np.float64) <= t
    _, b0 = ndimage.label(fg, structure=ndimage.generate_binary_structure(3, 1))
    bg = np.pad(~fg, 1, constant_values=True)
    _, nbg = ndimage.label(bg, structure=ndimage.generate_binary_structure(3, 3))
    return b0, nbg - 1


# ------------------------------------------------------------- soft by hand
def _sig(x):
    if x >= 0:
        return 1.0 / (1.0 + math.exp(-x))
    e = math.exp(x)
    return e / (1.0 + e)


def _cells_by_hand(g):
    """List of (value, dim) of every cell, enumerated with explicit loops."""
    out = []
    if g.ndim == 2:
        ny, nx = g.shape
        for y in range(ny):
            for x in range(nx):
                a = float(g[y, x])
                out.append((a, 0))
                if x + 1 < nx:
                    out.append((max(a, float(g[y, x + 1])), 1))
                if y + 1 < ny:
                    out.append((max(a, float(g[y + 1, x])), 1))
                if x + 1 < nx and y + 1 < ny:
                    out.append((max(a, float(g[y, x + 1]), float(g[y + 1, x]), float(g[y + 1, x + 1])), 2))
        return out
    nz, ny, nx = g.shape
    for z in range(nz):
        for y in range(ny):
            for x in range(nx):
                for dz in (0, 1):
                    for dy in (0, 1):
                        for dx in (0, 1):
                            if z + dz >= nz or y + dy >= ny or x + dx >= nx:
                                continue
                            vals = [float(g[z + a, y + b, x + c])
                                    for a in range(dz + 1) for b in range(dy + 1) for c in range(dx + 1)]
                            out.append((max(vals), dz + dy + dx))
    return out


def soft_by_hand(g, tau, lam):
    cells = _cells_by_hand(g)
    return [sum((-1) ** d * _sig(lam * (float(t) - v)) for v, d in cells) for t in tau]


def soft_bwd_by_hand(g, tau, lam, gout):
    cells = _cells_by_hand(g)
    res = []
    for t, gk in zip(tau, gout):
        acc = 0.0
        for v, d in cells:
            s = _sig(lam * (float(t) - v))
            acc += (-1) ** d * s * (1.0 - s)
        res.append(float(gk) * lam * acc)
    return res
