"""The C ABI on the CPU: the library loads, exports what include/ecc.h declares,
and rejects bad arguments with the documented status before touching a GPU."""

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ecc.h")


@pytest.fixture(scope="module")
def L():
    from euler_characteristic_curves_amd import _lib
    return _lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ecc_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted([
        "ecc_hard_2d", "ecc_hard_3d", "ecc_hard_3d_static", "ecc_hard_2d_batched", "ecc_hard_3d_batched",
        "ecc_soft_fwd", "ecc_soft_bwd_tau", "ecc_soft_bwd_grid",
        "ecc_soft_fwd_batched", "ecc_soft_bwd_tau_batched", "ecc_soft_bwd_tau_shared", "ecc_soft_bwd_grid_batched",
        "ecc_height", "ecc_height_bwd", "ecc_height_workspace_bytes",
        "ecc_workspace_bytes", "ecc_workspace_bytes_batched", "ecc_status_string", "ecc_last_error",
        "ecc_version"])


def test_library_exports_every_declared_symbol(L):
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(L.EXPORTS) == set(declared_functions())


def test_header_constants_match_binding(L):
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define\s+(ECC_\w+)\s+(\d+)\b", text))
    for name, val in consts.items():
        assert getattr(L, name) == int(val), name


def test_status_strings_and_version(L):
    for code in range(9):
        s = L.lib.ecc_status_string(code)
        assert s and s != b"unknown status"
    assert L.lib.ecc_status_string(99) == b"unknown status"
    assert L.lib.ecc_version() == b"0.1.0"


def test_workspace_bytes(L):
    f = L.lib.ecc_workspace_bytes
    assert f(0, 2, None, 0) == 0
    assert f(0, 2, None, 8193) == 0
    assert f(7, 2, None, 16) == 0
    small = f(0, 2, None, 1)
    assert small == f(1, 3, None, 256) == f(2, 3, None, 100) > 0
    assert f(0, 3, None, 8192) > small
    assert f(0, 3, None, 8192) % 8 == 0


def test_workspace_bytes_batched(L):
    f = L.lib.ecc_workspace_bytes_batched
    assert f(0, 0, 16) == 0 and f(0, 1, 0) == 0 and f(9, 1, 16) == 0
    one = f(0, 1, 256)
    assert one >= L.lib.ecc_workspace_bytes(0, 2, None, 256) and one % 256 == 0
    # grids of a large batch share the launch's workgroups: smaller slices
    assert f(0, 1000, 256) < 1000 * one
    assert f(0, 1000, 256) % 1000 == 0


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def hard2d(L, grid=FAKE, dtype=1, ny=4, nx=4, tau=FAKE, H=4, out=FAKE, ws=FAKE, wsb=1 << 30):
    return L.lib.ecc_hard_2d(grid, dtype, ny, nx, tau, H, out, ws, wsb, None)


def test_hard_argument_errors(L):
    assert hard2d(L, grid=None) == L.ECC_E_NULL
    assert b"grid" in L.lib.ecc_last_error()
    assert hard2d(L, tau=None) == L.ECC_E_NULL
    assert hard2d(L, out=None) == L.ECC_E_NULL
    assert hard2d(L, dtype=2) == L.ECC_E_DTYPE
    assert hard2d(L, dtype=-1) == L.ECC_E_DTYPE
    assert hard2d(L, ny=0) == L.ECC_E_SHAPE
    assert hard2d(L, nx=-3) == L.ECC_E_SHAPE
    assert hard2d(L, ny=1 << 30, nx=1 << 30) == L.ECC_E_SHAPE
    assert hard2d(L, H=0) == L.ECC_E_NTHRESH
    assert hard2d(L, H=8193) == L.ECC_E_NTHRESH
    assert hard2d(L, ws=None) == L.ECC_E_WORKSPACE
    assert hard2d(L, wsb=100) == L.ECC_E_WORKSPACE
    assert b"needs" in L.lib.ecc_last_error()
    r = L.lib.ecc_hard_3d(FAKE, 0, 0, 4, 4, FAKE, 4, FAKE, FAKE, 1 << 30, None)
    assert r == L.ECC_E_SHAPE
    r = L.lib.ecc_hard_3d(FAKE, 0, 1 << 14, 1 << 14, 1 << 14, FAKE, 4, FAKE, FAKE, 1 << 30, None)
    assert r == L.ECC_E_SHAPE


def hard_batched(L, B=3, nz=2, ny=4, nx=4, tau_stride=0, H=4, grid=FAKE, tau=FAKE, out=FAKE, ws=FAKE,
                 wsb=1 << 40, dtype=1):
    return L.lib.ecc_hard_3d_batched(grid, dtype, B, nz, ny, nx, tau, tau_stride, H, out, ws, wsb, None)


def test_hard_batched_argument_errors(L):
    assert hard_batched(L, grid=None) == L.ECC_E_NULL
    assert hard_batched(L, out=None) == L.ECC_E_NULL
    assert hard_batched(L, dtype=5) == L.ECC_E_DTYPE
    assert hard_batched(L, B=0) == L.ECC_E_SHAPE
    assert b"batch" in L.lib.ecc_last_error()
    assert hard_batched(L, B=-2) == L.ECC_E_SHAPE
    assert hard_batched(L, tau_stride=-1) == L.ECC_E_SHAPE
    assert hard_batched(L, nz=0) == L.ECC_E_SHAPE
    assert hard_batched(L, B=1 << 30, nz=1 << 6, ny=1 << 6, nx=1 << 6) == L.ECC_E_SHAPE
    assert hard_batched(L, H=0) == L.ECC_E_NTHRESH
    assert hard_batched(L, ws=None) == L.ECC_E_WORKSPACE
    need = L.lib.ecc_workspace_bytes_batched(0, 3, 4)
    assert hard_batched(L, wsb=need - 1) == L.ECC_E_WORKSPACE
    assert L.lib.ecc_hard_2d_batched(FAKE, 1, 0, 4, 4, FAKE, 0, 4, FAKE, FAKE, 1 << 40, None) == L.ECC_E_SHAPE


def soft(L, ndim=3, shape=(4, 4, 4), lam=1.0, H=4, grid=FAKE, tau=FAKE, out=FAKE, ws=FAKE, wsb=1 << 30,
         bwd=False, gout=FAKE):
    arr = (ctypes.c_int64 * max(1, len(shape)))(*shape) if shape is not None else None
    sp = ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None
    if bwd:
        return L.lib.ecc_soft_bwd_tau(grid, ndim, sp, tau, H, lam, gout, out, ws, wsb, None)
    return L.lib.ecc_soft_fwd(grid, ndim, sp, tau, H, lam, out, ws, wsb, None)


@pytest.mark.parametrize("bwd", [False, True])
def test_soft_argument_errors(L, bwd):
    assert soft(L, grid=None, bwd=bwd) == L.ECC_E_NULL
    assert soft(L, shape=None, bwd=bwd) == L.ECC_E_NULL
    assert soft(L, tau=None, bwd=bwd) == L.ECC_E_NULL
    assert soft(L, out=None, bwd=bwd) == L.ECC_E_NULL
    assert soft(L, ndim=4, shape=(2, 2, 2, 2), bwd=bwd) == L.ECC_E_SHAPE
    assert soft(L, ndim=1, shape=(5,), bwd=bwd) == L.ECC_E_SHAPE
    assert soft(L, shape=(4, 0, 4), bwd=bwd) == L.ECC_E_SHAPE
    for lam in (0.0, -1.0, math.inf, math.nan):
        assert soft(L, lam=lam, bwd=bwd) == L.ECC_E_LAMBDA
    assert soft(L, H=0, bwd=bwd) == L.ECC_E_NTHRESH
    assert soft(L, wsb=10, bwd=bwd) == L.ECC_E_WORKSPACE
    assert soft(L, ws=None, bwd=bwd) == L.ECC_E_WORKSPACE
    if bwd:
        assert soft(L, gout=None, bwd=True) == L.ECC_E_NULL


def soft_grid(L, ndim=3, shape=(4, 4, 4), lam=1.0, H=4, grid=FAKE, tau=FAKE, gout=FAKE, out=FAKE):
    arr = (ctypes.c_int64 * max(1, len(shape)))(*shape) if shape is not None else None
    sp = ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None
    return L.lib.ecc_soft_bwd_grid(grid, ndim, sp, tau, H, lam, gout, out, None)


def test_soft_grid_argument_errors(L):
    assert soft_grid(L, grid=None) == L.ECC_E_NULL
    assert soft_grid(L, shape=None) == L.ECC_E_NULL
    assert soft_grid(L, tau=None) == L.ECC_E_NULL
    assert soft_grid(L, out=None) == L.ECC_E_NULL
    assert soft_grid(L, gout=None) == L.ECC_E_NULL
    assert b"grad_out" in L.lib.ecc_last_error()
    assert soft_grid(L, ndim=4, shape=(2, 2, 2, 2)) == L.ECC_E_SHAPE
    assert soft_grid(L, ndim=2, shape=(0, 3)) == L.ECC_E_SHAPE
    assert soft_grid(L, shape=(1 << 14, 1 << 14, 1 << 14)) == L.ECC_E_SHAPE
    for lam in (0.0, -2.0, math.inf, math.nan):
        assert soft_grid(L, lam=lam) == L.ECC_E_LAMBDA
    assert soft_grid(L, H=0) == L.ECC_E_NTHRESH
    assert soft_grid(L, H=8193) == L.ECC_E_NTHRESH


@pytest.mark.parametrize("which", ["fwd", "bwd_tau", "bwd_tau_shared", "bwd_grid"])
def test_soft_batched_argument_errors(L, which):
    def call(B=2, ts=0, H=4, lam=1.0, ws=FAKE, wsb=1 << 40, gout=FAKE, shape=(4, 4, 4), grid=FAKE):
        arr = (ctypes.c_int64 * len(shape))(*shape)
        sp = ctypes.cast(arr, ctypes.c_void_p)
        if which == "fwd":
            return L.lib.ecc_soft_fwd_batched(grid, len(shape), sp, B, FAKE, ts, H, lam, FAKE, ws, wsb, None)
        if which == "bwd_tau":
            return L.lib.ecc_soft_bwd_tau_batched(grid, len(shape), sp, B, FAKE, ts, H, lam, gout, FAKE, ws, wsb,
                                                  None)
        if which == "bwd_tau_shared":  # no tau_stride: the thresholds are shared
            if ts < 0:
                return L.ECC_E_SHAPE
            return L.lib.ecc_soft_bwd_tau_shared(grid, len(shape), sp, B, FAKE, H, lam, gout, FAKE, ws, wsb, None)
        return L.lib.ecc_soft_bwd_grid_batched(grid, len(shape), sp, B, FAKE, ts, H, lam, gout, FAKE, None)
    assert call(grid=None) == L.ECC_E_NULL
    assert call(B=0) == L.ECC_E_SHAPE
    assert call(ts=-4) == L.ECC_E_SHAPE
    assert call(shape=(3, 0)) == L.ECC_E_SHAPE
    assert call(B=1 << 30, shape=(1 << 6, 1 << 6, 1 << 6)) == L.ECC_E_SHAPE
    assert call(lam=0.0) == L.ECC_E_LAMBDA
    assert call(H=0) == L.ECC_E_NTHRESH
    if which != "fwd":
        assert call(gout=None) == L.ECC_E_NULL
    if which != "bwd_grid":
        assert call(ws=None) == L.ECC_E_WORKSPACE
        assert call(wsb=L.lib.ecc_workspace_bytes_batched(1, 2, 4) - 1) == L.ECC_E_WORKSPACE


def test_height_argument_errors(L):
    def fwd(shape=(4, 5), D=2, grid=FAKE, dirs=FAKE, alpha=FAKE, out=FAKE):
        arr = (ctypes.c_int64 * len(shape))(*shape)
        return L.lib.ecc_height(grid, len(shape), ctypes.cast(arr, ctypes.c_void_p), dirs, alpha, D, out, None)

    def bwd(shape=(4, 5), D=2, gg=FAKE, gd=FAKE, ga=FAKE, ws=FAKE, wsb=1 << 30):
        arr = (ctypes.c_int64 * len(shape))(*shape)
        return L.lib.ecc_height_bwd(FAKE, len(shape), ctypes.cast(arr, ctypes.c_void_p), FAKE, FAKE, D, gg, gd, ga,
                                    ws, wsb, None)
    assert fwd(grid=None) == L.ECC_E_NULL
    assert fwd(dirs=None) == L.ECC_E_NULL
    assert fwd(alpha=None) == L.ECC_E_NULL
    assert fwd(out=None) == L.ECC_E_NULL
    assert fwd(shape=(2, 2, 2, 2)) == L.ECC_E_SHAPE
    assert fwd(shape=(0, 5)) == L.ECC_E_SHAPE
    assert fwd(shape=(3, (1 << 24) + 1)) == L.ECC_E_SHAPE
    assert fwd(D=0) == L.ECC_E_NDIRS
    assert fwd(D=4097) == L.ECC_E_NDIRS
    assert fwd(shape=(1 << 20, 1 << 20), D=2) == L.ECC_E_SHAPE
    assert bwd(gg=None, gd=None, ga=None) == L.ECC_E_NULL
    assert bwd(ga=None) == L.ECC_E_NULL
    assert bwd(ws=None) == L.ECC_E_WORKSPACE
    assert bwd(wsb=L.lib.ecc_height_workspace_bytes(2, 2) - 1) == L.ECC_E_WORKSPACE
    assert L.lib.ecc_height_workspace_bytes(4, 2) == 0 and L.lib.ecc_height_workspace_bytes(2, 0) == 0
    assert L.lib.ecc_height_workspace_bytes(3, 4096) > 0


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    import euler_characteristic_curves_amd as E
    g = torch.zeros((4, 4))
    with pytest.raises(ValueError):
        E.ecc_hard_2d(g, torch.zeros(4))
    with pytest.raises(ValueError):
        E.ecc_soft_fwd(g, torch.zeros(4), 1.0)


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "euler_characteristic_curves_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "oracle/" not in text, f
