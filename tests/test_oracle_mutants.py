"""Planted mistakes in the oracle must be caught by the pins.

Each mutant swaps one internal step of the CPU oracle for a plausible wrong
version (a dropped cell type, a wrong sign, a wrong corner, a strict
comparison, a shifted prefix sum, a transposed axis) and checks that the
brute-force / topology pins reject it.  Mistakes are planted only in the
oracle, on the CPU.
"""

import itertools

import numpy as np
import pytest

import oracle
from oracle import ecc as oecc
from tests import pins

_real_cell_values = oecc.cell_values
_real_first_k = oecc.first_k_bins


def _cells_mutant(kind):
    def gen(grid):
        grid = np.asarray(grid)
        cells = list(_real_cell_values(grid))
        exts = [e for e in itertools.product((0, 1), repeat=grid.ndim)
                if min(n - x for n, x in zip(grid.shape, e)) > 0]
        for (val, dim), ext in zip(cells, exts):
            if kind == "drop_top" and dim == grid.ndim:
                continue
            if kind == "edge_sign" and dim == 1:
                yield val, 0
                continue
            if kind == "min_not_max" and dim == 1:
                # an edge valued by its lower corner
                anchors = [n - e for n, e in zip(grid.shape, ext)]
                a = grid[tuple(slice(0, s) for s in anchors)]
                b = grid[tuple(slice(e, e + s) for e, s in zip(ext, anchors))]
                yield np.minimum(a, b), dim
                continue
            if kind == "square_misses_corner" and dim == 2:
                # a square valued without its far corner
                anchors = [n - e for n, e in zip(grid.shape, ext)]
                axes = [i for i, e in enumerate(ext) if e]
                v = grid[tuple(slice(0, s) for s in anchors)]
                for ax in axes:
                    off = [0] * grid.ndim
                    off[ax] = 1
                    v = np.maximum(v, grid[tuple(slice(o, o + s) for o, s in zip(off, anchors))])
                yield v, dim
                continue
            if kind == "transposed" and dim == 1 and ext[-1] == 0:
                # edges along another axis valued with the x neighbour (swapped axis)
                if grid.shape[-1] > 1:
                    yield np.maximum(grid[..., :-1], grid[..., 1:]), dim
                continue
            yield val, dim
    return gen


def _strict_bins(values, tau):
    t = np.asarray(tau).astype(np.float32).astype(np.float64)
    return np.searchsorted(t, np.asarray(values, np.float64).ravel(), side="right").astype(np.int64)


def _run_pins():
    """Return True if every pin passes for the currently patched oracle."""
    rng = np.random.default_rng(1234)
    try:
        for ndim in (2, 3):
            for _ in range(12):
                shape = tuple(int(s) for s in rng.integers(2, 6, size=ndim))
                g = rng.integers(0, 4, size=shape).astype(np.float32)
                tau = np.array([-1, 0, 1, 2, 3, 4], np.float32)
                got = oracle.ecc_hard(g, tau)
                if got.tolist() != [pins.brute_chi(g, float(t)) for t in tau]:
                    return False
                for t in (0.0, 1.0, 2.0):
                    if oracle.ecc_at(g, t) != pins.brute_chi(g, t):
                        return False
        for _ in range(12):
            g = rng.integers(0, 3, size=(5, 7)).astype(np.float32)
            for t in (0.0, 1.0):
                b0, b1 = pins.betti_2d(g, t)
                if oracle.ecc_at(g, t) != b0 - b1:
                    return False
    except Exception:
        return False
    return True


def test_unpatched_oracle_passes_pins():
    assert _run_pins()


@pytest.mark.parametrize("kind", ["drop_top", "edge_sign", "min_not_max", "square_misses_corner", "transposed"])
def test_cell_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(oecc, "cell_values", _cells_mutant(kind))
    assert not _run_pins()


def test_strict_comparison_is_caught(monkeypatch):
    monkeypatch.setattr(oecc, "first_k_bins", _strict_bins)
    assert not _run_pins()


def test_shifted_prefix_sum_is_caught(monkeypatch):
    real = oecc.ecc_hard

    def shifted(grid, tau, slab=32):
        e = real(grid, tau, slab)
        return np.concatenate([[0], e[:-1]])

    monkeypatch.setattr(oracle, "ecc_hard", shifted)
    assert not _run_pins()


def test_soft_sign_mutant_is_caught(monkeypatch):
    """A soft oracle that drops the sign of edges fails the constant-grid closed form."""
    def bad_grouped(grid, slab=32):
        u, w = [], []
        for val, dim in _real_cell_values(grid):
            u.append(val.astype(np.float64).ravel())
            w.append(np.ones(val.size, np.int64))
        return np.concatenate(u), np.concatenate(w)

    monkeypatch.setattr(oecc, "_grouped_weights", bad_grouped)
    g = np.full((3, 4), 0.5, np.float32)
    tau = np.array([0.25, 0.5, 0.75], np.float32)
    want = [pins._sig(10.0 * (float(t) - 0.5)) for t in tau]
    assert not np.allclose(oracle.ecc_soft(g, tau, 10.0), want)


# ---------------------------------------------------- grid gradient mutants
def _grad_mutant(kind):
    """ecc_soft_bwd_grid with one planted mistake."""
    def f(grid, tau, lam, grad_out):
        grid, t, lam, g = oecc._grad_inputs(grid, tau, lam, grad_out)
        X = grid.astype(np.float64)
        index = np.arange(X.size).reshape(X.shape)
        out = np.zeros(X.size)
        for ext in itertools.product((0, 1), repeat=X.ndim):
            anchors = [n - e for n, e in zip(X.shape, ext)]
            if min(anchors) <= 0:
                continue
            offs = list(itertools.product(*[range(e + 1) for e in ext]))
            if kind == "last_index_ties":
                offs = offs[::-1]
            vals = np.stack([X[tuple(slice(o, o + a) for o, a in zip(off, anchors))] for off in offs])
            idxs = np.stack([index[tuple(slice(o, o + a) for o, a in zip(off, anchors))] for off in offs])
            am = np.argmax(vals, axis=0)
            v = np.take_along_axis(vals, am[None], 0)[0].ravel()
            tgt = np.take_along_axis(idxs, am[None], 0)[0].ravel()
            if kind == "to_anchor":
                tgt = idxs[0].ravel()
            sign = 1 if kind == "no_dim_sign" else (-1) ** sum(ext)
            lam_f = 1.0 if kind == "no_lambda" else lam
            pre = lam_f if kind == "plus_sign" else -lam_f
            np.add.at(out, tgt, pre * sign * oecc._h_of(v, t, lam, g))
        return out.reshape(X.shape)
    return f


def _run_grad_pins():
    """Finite differences of the by-hand forward, the constant-grid closed form
    and the sum rule; True if the current oracle.ecc_soft_bwd_grid passes all."""
    rng = np.random.default_rng(4321)
    lam = 9.0
    tau = np.linspace(-0.1, 1.1, 7).astype(np.float32)
    gout = rng.standard_normal(7).astype(np.float32)
    for shape in ((3, 4), (2, 3, 3)):
        n = int(np.prod(shape))
        g = (rng.permutation(n) / n).reshape(shape)
        got = oracle.ecc_soft_bwd_grid(g, tau, lam, gout)
        h = 1e-6
        for p in np.ndindex(*shape):
            up, dn = g.copy(), g.copy()
            up[p] += h
            dn[p] -= h
            fd = float(np.dot(gout.astype(np.float64),
                              np.subtract(pins.soft_by_hand(up, tau, lam), pins.soft_by_hand(dn, tau, lam)))) / (2 * h)
            if abs(fd - got[p]) > 1e-6 * max(1.0, abs(got[p])):
                return False
        c = np.full(shape, 0.5, np.float32)
        want = np.zeros(shape)
        want[tuple(s - 1 for s in shape)] = -lam * sum(
            float(gk) * pins._sig(lam * (float(t) - 0.5)) * (1 - pins._sig(lam * (float(t) - 0.5)))
            for t, gk in zip(tau, gout))
        if not np.allclose(oracle.ecc_soft_bwd_grid(c, tau, lam, gout), want, rtol=1e-12, atol=1e-15):
            return False
        q = (rng.integers(0, 3, shape) / 2).astype(np.float32)
        s = oracle.ecc_soft_bwd_grid(q, tau, lam, gout).sum()
        if abs(s + oracle.ecc_soft_bwd_tau(q, tau, lam, gout).sum()) > 1e-9:
            return False
    return True


def test_unpatched_grid_gradient_passes_pins():
    assert _run_grad_pins()


@pytest.mark.parametrize("kind", ["last_index_ties", "to_anchor", "no_dim_sign", "no_lambda", "plus_sign"])
def test_grid_gradient_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(oracle, "ecc_soft_bwd_grid", _grad_mutant(kind))
    assert not _run_grad_pins()


# ------------------------------------------------- directional height mutants
def test_height_axis_order_mutant_is_caught(monkeypatch):
    """Heights with the axes taken fastest first fail the hand-worked values."""
    real = oecc.height_values

    def reversed_axes(grid, dirs, alpha):
        X = np.asarray(grid, np.float32)
        U = np.asarray(dirs, np.float32).reshape(-1, X.ndim)[:, ::-1]
        return real(X, U, alpha)

    monkeypatch.setattr(oracle, "height_values", reversed_axes)
    from tests import test_oracle_pins as P
    with pytest.raises(AssertionError):
        P.test_height_values_by_hand()


def test_height_bwd_without_alpha_is_caught(monkeypatch):
    """A backward that forgets alpha in dL/du fails the finite differences."""
    real = oecc.height_bwd

    def no_alpha(grad_h, dirs, alpha):
        dX, dU, dA = real(grad_h, dirs, alpha)
        a = np.asarray(alpha, np.float32).astype(np.float64).reshape(-1, 1)
        return dX, dU / a, dA

    monkeypatch.setattr(oracle, "height_bwd", no_alpha)
    from tests import test_oracle_pins as P
    with pytest.raises(AssertionError):
        P.test_height_gradient_finite_differences((4, 5))


# --------------------------------------- checkers of several thresholds
# The checkers of sampled outputs on large grids, each rewritten with one
# planted mistake; the pins in test_oracle_pins.py must reject every one.
def _at_many_mutant(kind):
    def f(grid, ts, slab=32):
        grid = oecc._check_grid(grid)
        t = np.asarray(ts, dtype=np.float32).astype(np.float64).ravel()
        chi = np.zeros(t.size, dtype=np.int64)
        for sub, keep in oecc._z_slabs(grid, slab):
            if kind == "halo_twice":
                keep = None
            for val, dim in oecc._slab_cells(sub, keep):
                v = val.astype(np.float64)
                for i, ti in enumerate(t):
                    n = np.count_nonzero(v < ti) if kind == "strict" else np.count_nonzero(v <= ti)
                    sign = 1 if (kind == "no_sign" and dim == 1) else (-1) ** dim
                    chi[i] += sign * int(n)
        return chi
    return f


def _soft_many_mutant(kind, bwd):
    def f(grid, ts, lam, *rest, slab=32):
        t = np.asarray(ts, dtype=np.float32).astype(np.float64).ravel()
        lam = oecc._check_lambda(lam)
        acc = np.zeros(t.size, dtype=np.float64)
        for sub, keep in oecc._z_slabs(oecc._check_grid(grid), slab):
            if kind == "halo_twice":
                keep = None
            for val, dim in oecc._slab_cells(sub, keep):
                v = val.astype(np.float64)
                sign = 1 if kind == "no_sign" else (-1) ** dim
                for i, ti in enumerate(t):
                    x = (ti - v) if kind == "no_lambda_inside" else lam * (ti - v)
                    acc[i] += sign * float((oecc._dsig(x) if bwd else oecc.sigmoid(x)).sum())
        if not bwd:
            return acc
        g = np.asarray(rest[0], dtype=np.float32).astype(np.float64).ravel()
        if kind == "g_reversed":
            g = g[::-1]
        scale = 1.0 if kind == "no_lambda" else lam
        return g * scale * acc
    return f


@pytest.mark.parametrize("kind", ["strict", "halo_twice", "no_sign"])
def test_at_many_mutants_are_caught(monkeypatch, kind):
    from tests import test_oracle_pins as P
    monkeypatch.setattr(oracle, "ecc_at_many", _at_many_mutant(kind))
    with pytest.raises(AssertionError):
        P.check_at_many()


@pytest.mark.parametrize("kind", ["no_sign", "halo_twice", "no_lambda_inside"])
def test_soft_at_many_mutants_are_caught(monkeypatch, kind):
    from tests import test_oracle_pins as P
    monkeypatch.setattr(oracle, "ecc_soft_at_many", _soft_many_mutant(kind, bwd=False))
    with pytest.raises(AssertionError):
        P.check_soft_at_many()


@pytest.mark.parametrize("kind", ["no_sign", "halo_twice", "no_lambda", "no_lambda_inside", "g_reversed"])
def test_soft_bwd_at_many_mutants_are_caught(monkeypatch, kind):
    from tests import test_oracle_pins as P
    monkeypatch.setattr(oracle, "ecc_soft_bwd_at_many", _soft_many_mutant(kind, bwd=True))
    with pytest.raises(AssertionError):
        P.check_soft_bwd_at_many()


@pytest.mark.parametrize("name", ["ecc_at_many", "ecc_soft_at_many", "ecc_soft_bwd_at_many"])
def test_many_mutant_builders_reproduce_the_oracle_unplanted(monkeypatch, name):
    """The rewrites above, with nothing planted, pass the same pins, so each
    mutant fails only because of its planted mistake."""
    from tests import test_oracle_pins as P
    if name == "ecc_at_many":
        monkeypatch.setattr(oracle, name, _at_many_mutant("none"))
        P.check_at_many()
    elif name == "ecc_soft_at_many":
        monkeypatch.setattr(oracle, name, _soft_many_mutant("none", bwd=False))
        P.check_soft_at_many()
    else:
        monkeypatch.setattr(oracle, name, _soft_many_mutant("none", bwd=True))
        P.check_soft_bwd_at_many()
