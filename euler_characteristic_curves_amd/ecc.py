"""Thin PyTorch binding of libecc_mi355 (argument marshalling only).

Every function here takes torch tensors that live on a ROCm device, checks
their dtype / layout, and calls the C entry point of the same name on the
current torch stream.  All arithmetic happens in the HIP kernels.
"""

import ctypes

import torch

from . import _lib
from ._lib import EccError, check, lib

__all__ = [
    "ecc_hard_2d", "ecc_hard_3d", "ecc_hard", "ecc_hard_batched", "ecc_soft_fwd", "ecc_soft_bwd_tau",
    "ecc_soft_bwd_grid", "ecc_soft_fwd_batched", "ecc_soft_bwd_tau_batched", "ecc_soft_bwd_grid_batched",
    "workspace_bytes", "workspace_bytes_batched", "get_workspace", "EccError", "SoftECC", "soft_ecc",
]

_WS = {}
_WS_BYTES = {}


def workspace_bytes(op, H, shape=None):
    key = (op, len(shape) if shape else 0, int(H))
    n = _WS_BYTES.get(key)
    if n is None:
        n = int(lib.ecc_workspace_bytes(op, key[1], None, key[2]))
        if n == 0:
            raise EccError(_lib.ECC_E_NTHRESH, f"no workspace size for op={op} H={H}")
        _WS_BYTES[key] = n
    return n


def workspace_bytes_batched(op, batch, H):
    n = lib.ecc_workspace_bytes_batched(op, int(batch), int(H))
    if n == 0:
        raise EccError(_lib.ECC_E_NTHRESH, f"no workspace size for op={op} batch={batch} H={H}")
    return int(n)


def get_workspace(nbytes, device, stream):
    """A zero-filled workspace of >= nbytes for this device and stream.

    The library leaves a workspace zero-filled after every call, so one
    buffer per (device, stream) is reused; calls on one stream never overlap.
    """
    key = (device.index, int(stream.cuda_stream))
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        if isinstance(stream, torch.cuda.Stream):
            with torch.cuda.stream(stream):
                ws = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
        else:  # the caller's current stream, which is where torch allocates
            ws = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
        _WS[key] = ws
    return ws


class _CurrentStream:
    """The caller's current stream as its raw handle (``.cuda_stream``)."""

    __slots__ = ("cuda_stream",)

    def __init__(self, handle):
        self.cuda_stream = handle


# torch's raw current-stream query costs ~0.1 us against ~2 us for building a
# Stream object, which dominates the host time of a call on a small grid
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t):
    if _raw_current_stream is not None:
        return _CurrentStream(_raw_current_stream(t.get_device()))
    return torch.cuda.current_stream(t.device)


def _grid_dtype(grid):
    if grid.dtype == torch.uint8:
        return _lib.ECC_U8
    if grid.dtype == torch.float32:
        return _lib.ECC_F32
    raise TypeError(f"grid dtype {grid.dtype} not supported (uint8 or float32)")


def _dev_tensor(t, name, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a ROCm device (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return t.data_ptr()  # an int: the argtypes (c_void_p) convert it


def ecc_hard_3d_static(grid, tau, out):
    """ecc_hard_3d on the library's static scratch array: no workspace and no
    allocation by the library (see include/ecc.h); ``out`` is caller-owned int64[H]."""
    _dev_tensor(grid, "grid")
    if grid.dim() not in (2, 3):
        raise ValueError("grid must be 2D or 3D")
    _dev_tensor(tau, "tau", torch.float32, grid.device)
    H = tau.numel()
    _dev_tensor(out, "out", torch.int64, grid.device)
    if tuple(out.shape) != (H,):
        raise ValueError("out must be [H]")
    dims = (1,) + tuple(grid.shape) if grid.dim() == 2 else tuple(grid.shape)
    check(lib.ecc_hard_3d_static(_ptr(grid), _grid_dtype(grid), *dims, _ptr(tau), H, _ptr(out),
                                 _stream(grid).cuda_stream), "ecc_hard_3d_static")
    return out


def ecc_hard_2d(grid, tau, out=None, ws=None):
    """Hard ECC of a 2D uint8/float32 grid: int64[H] (see include/ecc.h)."""
    _dev_tensor(grid, "grid")
    if grid.dim() != 2:
        raise ValueError("grid must be 2D")
    _dev_tensor(tau, "tau", torch.float32, grid.device)
    H = tau.numel()
    if out is None:
        out = torch.empty(H, dtype=torch.int64, device=grid.device)
    _dev_tensor(out, "out", torch.int64, grid.device)
    s = _stream(grid)
    nb = workspace_bytes(_lib.ECC_OP_HARD, H)
    ws = get_workspace(nb, grid.device, s) if ws is None else ws
    check(lib.ecc_hard_2d(_ptr(grid), _grid_dtype(grid), grid.shape[0], grid.shape[1], _ptr(tau), H,
                          _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                          s.cuda_stream), "ecc_hard_2d")
    return out


def ecc_hard_3d(grid, tau, out=None, ws=None):
    """Hard ECC of a 3D uint8/float32 grid: int64[H] (see include/ecc.h)."""
    _dev_tensor(grid, "grid")
    if grid.dim() != 3:
        raise ValueError("grid must be 3D")
    _dev_tensor(tau, "tau", torch.float32, grid.device)
    H = tau.numel()
    if out is None:
        out = torch.empty(H, dtype=torch.int64, device=grid.device)
    _dev_tensor(out, "out", torch.int64, grid.device)
    s = _stream(grid)
    nb = workspace_bytes(_lib.ECC_OP_HARD, H)
    ws = get_workspace(nb, grid.device, s) if ws is None else ws
    check(lib.ecc_hard_3d(_ptr(grid), _grid_dtype(grid), grid.shape[0], grid.shape[1], grid.shape[2],
                          _ptr(tau), H, _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                          s.cuda_stream), "ecc_hard_3d")
    return out


def ecc_hard(grid, tau, out=None, ws=None):
    """Dispatch on grid.dim(): ecc_hard_2d or ecc_hard_3d."""
    if grid.dim() == 2:
        return ecc_hard_2d(grid, tau, out, ws)
    if grid.dim() == 3:
        return ecc_hard_3d(grid, tau, out, ws)
    raise ValueError("grid must be 2D or 3D")


def ecc_hard_batched(grids, tau, out=None, ws=None):
    """Hard ECC of a batch of grids [B, ny, nx] or [B, nz, ny, nx]: int64[B, H].

    ``tau`` is float32[H] (shared by every grid) or float32[B, H] (one row per
    grid); see ecc_hard_2d_batched / ecc_hard_3d_batched in include/ecc.h.
    """
    _dev_tensor(grids, "grids")
    if grids.dim() not in (3, 4):
        raise ValueError("grids must be [B, ny, nx] or [B, nz, ny, nx]")
    _dev_tensor(tau, "tau", torch.float32, grids.device)
    B = grids.shape[0]
    if tau.dim() == 1:
        H, tau_stride = tau.numel(), 0
    elif tau.dim() == 2 and tau.shape[0] == B:
        H, tau_stride = tau.shape[1], tau.shape[1]
    else:
        raise ValueError("tau must be [H] or [B, H]")
    if out is None:
        out = torch.empty((B, H), dtype=torch.int64, device=grids.device)
    _dev_tensor(out, "out", torch.int64, grids.device)
    if tuple(out.shape) != (B, H):
        raise ValueError("out must be [B, H]")
    s = _stream(grids)
    nb = workspace_bytes_batched(_lib.ECC_OP_HARD, B, H)
    ws = get_workspace(nb, grids.device, s) if ws is None else ws
    args = (_ptr(tau), tau_stride, H, _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
            s.cuda_stream)
    if grids.dim() == 3:
        check(lib.ecc_hard_2d_batched(_ptr(grids), _grid_dtype(grids), B, grids.shape[1], grids.shape[2], *args),
              "ecc_hard_2d_batched")
    else:
        check(lib.ecc_hard_3d_batched(_ptr(grids), _grid_dtype(grids), B, grids.shape[1], grids.shape[2],
                                      grids.shape[3], *args), "ecc_hard_3d_batched")
    return out


def _shape_arr(grid):
    if grid.dim() not in (2, 3):
        raise ValueError("grid must be 2D or 3D")
    return (ctypes.c_int64 * grid.dim())(*grid.shape)


def ecc_soft_fwd(grid, tau, lam, out=None, ws=None):
    """Soft ECC forward, float32[H] (see include/ecc.h)."""
    _dev_tensor(grid, "grid", torch.float32)
    _dev_tensor(tau, "tau", torch.float32, grid.device)
    H = tau.numel()
    if out is None:
        out = torch.empty(H, dtype=torch.float32, device=grid.device)
    _dev_tensor(out, "out", torch.float32, grid.device)
    shp = _shape_arr(grid)
    s = _stream(grid)
    nb = workspace_bytes(_lib.ECC_OP_SOFT_FWD, H)
    ws = get_workspace(nb, grid.device, s) if ws is None else ws
    check(lib.ecc_soft_fwd(_ptr(grid), grid.dim(), ctypes.cast(shp, ctypes.c_void_p), _ptr(tau), H,
                           float(lam), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                           s.cuda_stream), "ecc_soft_fwd")
    return out


def ecc_soft_bwd_tau(grid, tau, lam, grad_out, grad_tau=None, ws=None):
    """dL/dtau of the soft ECC, float32[H] (see include/ecc.h)."""
    _dev_tensor(grid, "grid", torch.float32)
    _dev_tensor(tau, "tau", torch.float32, grid.device)
    _dev_tensor(grad_out, "grad_out", torch.float32, grid.device)
    H = tau.numel()
    if grad_out.numel() != H:
        raise ValueError("grad_out must have H elements")
    if grad_tau is None:
        grad_tau = torch.empty(H, dtype=torch.float32, device=grid.device)
    _dev_tensor(grad_tau, "grad_tau", torch.float32, grid.device)
    shp = _shape_arr(grid)
    s = _stream(grid)
    nb = workspace_bytes(_lib.ECC_OP_SOFT_BWD, H)
    ws = get_workspace(nb, grid.device, s) if ws is None else ws
    check(lib.ecc_soft_bwd_tau(_ptr(grid), grid.dim(), ctypes.cast(shp, ctypes.c_void_p), _ptr(tau), H,
                               float(lam), _ptr(grad_out), _ptr(grad_tau), _ptr(ws),
                               ws.numel() * ws.element_size(), s.cuda_stream),
          "ecc_soft_bwd_tau")
    return grad_tau


def ecc_soft_bwd_grid(grid, tau, lam, grad_out, grad_grid=None):
    """dL/dgrid of the soft ECC, float32 of the grid's shape (see include/ecc.h)."""
    _dev_tensor(grid, "grid", torch.float32)
    _dev_tensor(tau, "tau", torch.float32, grid.device)
    _dev_tensor(grad_out, "grad_out", torch.float32, grid.device)
    H = tau.numel()
    if grad_out.numel() != H:
        raise ValueError("grad_out must have H elements")
    if grad_grid is None:
        grad_grid = torch.empty_like(grid)
    _dev_tensor(grad_grid, "grad_grid", torch.float32, grid.device)
    if grad_grid.shape != grid.shape:
        raise ValueError("grad_grid must have the grid's shape")
    shp = _shape_arr(grid)
    s = _stream(grid)
    check(lib.ecc_soft_bwd_grid(_ptr(grid), grid.dim(), ctypes.cast(shp, ctypes.c_void_p), _ptr(tau), H,
                                float(lam), _ptr(grad_out), _ptr(grad_grid), s.cuda_stream),
          "ecc_soft_bwd_grid")
    return grad_grid


class SoftECC(torch.autograd.Function):
    """Autograd wrapper: soft ECC, differentiable in the thresholds and the grid."""

    @staticmethod
    def forward(ctx, grid, tau, lam):
        ctx.save_for_backward(grid, tau)
        ctx.lam = float(lam)
        return ecc_soft_fwd(grid.detach().contiguous(), tau.detach().contiguous(), lam)

    @staticmethod
    def backward(ctx, grad_out):
        grid, tau = ctx.saved_tensors
        grid = grid.detach().contiguous()
        tau = tau.detach().contiguous()
        grad_out = grad_out.contiguous()
        g_grid = ecc_soft_bwd_grid(grid, tau, ctx.lam, grad_out) if ctx.needs_input_grad[0] else None
        g_tau = ecc_soft_bwd_tau(grid, tau, ctx.lam, grad_out) if ctx.needs_input_grad[1] else None
        return g_grid, g_tau, None


def soft_ecc(grid, tau, lam):
    """Soft ECC as an autograd op (differentiable in the grid and in tau)."""
    return SoftECC.apply(grid, tau, lam)


# ------------------------------------------------------------ soft batches
def _batch_args(grids, tau):
    _dev_tensor(grids, "grids", torch.float32)
    if grids.dim() not in (3, 4):
        raise ValueError("grids must be [B, ny, nx] or [B, nz, ny, nx]")
    _dev_tensor(tau, "tau", torch.float32, grids.device)
    B = grids.shape[0]
    if tau.dim() == 1:
        H, tau_stride = tau.numel(), 0
    elif tau.dim() == 2 and tau.shape[0] == B:
        H, tau_stride = tau.shape[1], tau.shape[1]
    else:
        raise ValueError("tau must be [H] or [B, H]")
    shp = (ctypes.c_int64 * (grids.dim() - 1))(*grids.shape[1:])
    return B, H, tau_stride, shp


def ecc_soft_fwd_batched(grids, tau, lam, out=None, ws=None):
    """Soft ECC of each grid of a batch: float32[B, H] (see include/ecc.h)."""
    B, H, ts, shp = _batch_args(grids, tau)
    if out is None:
        out = torch.empty((B, H), dtype=torch.float32, device=grids.device)
    _dev_tensor(out, "out", torch.float32, grids.device)
    if tuple(out.shape) != (B, H):
        raise ValueError("out must be [B, H]")
    s = _stream(grids)
    nb = workspace_bytes_batched(_lib.ECC_OP_SOFT_FWD, B, H)
    ws = get_workspace(nb, grids.device, s) if ws is None else ws
    check(lib.ecc_soft_fwd_batched(_ptr(grids), grids.dim() - 1, ctypes.cast(shp, ctypes.c_void_p), B,
                                   _ptr(tau), ts, H, float(lam), _ptr(out), _ptr(ws),
                                   ws.numel() * ws.element_size(), s.cuda_stream),
          "ecc_soft_fwd_batched")
    return out


def ecc_soft_bwd_tau_batched(grids, tau, lam, grad_out, grad_tau=None, ws=None):
    """Per-grid dL/dtau of a batch, float32[B, H] (see include/ecc.h)."""
    B, H, ts, shp = _batch_args(grids, tau)
    _dev_tensor(grad_out, "grad_out", torch.float32, grids.device)
    if tuple(grad_out.shape) != (B, H):
        raise ValueError("grad_out must be [B, H]")
    if grad_tau is None:
        grad_tau = torch.empty((B, H), dtype=torch.float32, device=grids.device)
    _dev_tensor(grad_tau, "grad_tau", torch.float32, grids.device)
    if tuple(grad_tau.shape) != (B, H):
        raise ValueError("grad_tau must be [B, H]")
    s = _stream(grids)
    nb = workspace_bytes_batched(_lib.ECC_OP_SOFT_BWD, B, H)
    ws = get_workspace(nb, grids.device, s) if ws is None else ws
    check(lib.ecc_soft_bwd_tau_batched(_ptr(grids), grids.dim() - 1, ctypes.cast(shp, ctypes.c_void_p), B,
                                       _ptr(tau), ts, H, float(lam), _ptr(grad_out), _ptr(grad_tau), _ptr(ws),
                                       ws.numel() * ws.element_size(), s.cuda_stream),
          "ecc_soft_bwd_tau_batched")
    return grad_tau


def ecc_soft_bwd_tau_shared(grids, tau, lam, grad_out, grad_tau=None, ws=None):
    """dL/dtau of one threshold array shared by a batch, summed over the batch on
    the device: float32[H] (see include/ecc.h)."""
    B, H, ts, shp = _batch_args(grids, tau)
    if ts != 0:
        raise ValueError("tau must be one [H] array shared by the batch")
    _dev_tensor(grad_out, "grad_out", torch.float32, grids.device)
    if tuple(grad_out.shape) != (B, H):
        raise ValueError("grad_out must be [B, H]")
    if grad_tau is None:
        grad_tau = torch.empty(H, dtype=torch.float32, device=grids.device)
    _dev_tensor(grad_tau, "grad_tau", torch.float32, grids.device)
    if tuple(grad_tau.shape) != (H,):
        raise ValueError("grad_tau must be [H]")
    s = _stream(grids)
    nb = workspace_bytes_batched(_lib.ECC_OP_SOFT_BWD, B, H)
    ws = get_workspace(nb, grids.device, s) if ws is None else ws
    check(lib.ecc_soft_bwd_tau_shared(_ptr(grids), grids.dim() - 1, ctypes.cast(shp, ctypes.c_void_p), B,
                                      _ptr(tau), H, float(lam), _ptr(grad_out), _ptr(grad_tau), _ptr(ws),
                                      ws.numel() * ws.element_size(), s.cuda_stream),
          "ecc_soft_bwd_tau_shared")
    return grad_tau


def ecc_soft_bwd_grid_batched(grids, tau, lam, grad_out, grad_grid=None):
    """dL/dgrids of a batch, float32 of the grids' shape (see include/ecc.h)."""
    B, H, ts, shp = _batch_args(grids, tau)
    _dev_tensor(grad_out, "grad_out", torch.float32, grids.device)
    if tuple(grad_out.shape) != (B, H):
        raise ValueError("grad_out must be [B, H]")
    if grad_grid is None:
        grad_grid = torch.empty_like(grids)
    _dev_tensor(grad_grid, "grad_grid", torch.float32, grids.device)
    if grad_grid.shape != grids.shape:
        raise ValueError("grad_grid must have the grids' shape")
    s = _stream(grids)
    check(lib.ecc_soft_bwd_grid_batched(_ptr(grids), grids.dim() - 1, ctypes.cast(shp, ctypes.c_void_p), B,
                                        _ptr(tau), ts, H, float(lam), _ptr(grad_out), _ptr(grad_grid),
                                        s.cuda_stream),
          "ecc_soft_bwd_grid_batched")
    return grad_grid


class SoftECCBatched(torch.autograd.Function):
    """Autograd wrapper over a batch: grids [B, ...], tau [H] (shared) or [B, H] -> [B, H]."""

    @staticmethod
    def forward(ctx, grids, tau, lam):
        ctx.save_for_backward(grids, tau)
        ctx.lam = float(lam)
        return ecc_soft_fwd_batched(grids.detach().contiguous(), tau.detach().contiguous(), lam)

    @staticmethod
    def backward(ctx, grad_out):
        grids, tau = ctx.saved_tensors
        grids = grids.detach().contiguous()
        tau_c = tau.detach().contiguous()
        grad_out = grad_out.contiguous()
        g_grid = g_tau = None
        if ctx.needs_input_grad[0]:
            g_grid = ecc_soft_bwd_grid_batched(grids, tau_c, ctx.lam, grad_out)
        if ctx.needs_input_grad[1]:
            if tau.dim() == 1:  # one threshold array shared by every grid: summed on the device
                g_tau = ecc_soft_bwd_tau_shared(grids, tau_c, ctx.lam, grad_out)
            else:
                g_tau = ecc_soft_bwd_tau_batched(grids, tau_c, ctx.lam, grad_out)
        return g_grid, g_tau, None


def soft_ecc_batched(grids, tau, lam):
    """Soft ECC of a batch of grids as an autograd op (differentiable in grids and tau)."""
    return SoftECCBatched.apply(grids, tau, lam)


# ----------------------------------------------------- directional heights
def _height_args(grid, dirs, alpha):
    _dev_tensor(grid, "grid", torch.float32)
    if grid.dim() not in (2, 3):
        raise ValueError("grid must be 2D or 3D")
    _dev_tensor(dirs, "dirs", torch.float32, grid.device)
    _dev_tensor(alpha, "alpha", torch.float32, grid.device)
    if dirs.dim() != 2 or dirs.shape[1] != grid.dim():
        raise ValueError("dirs must be [D, grid.dim()]")
    D = dirs.shape[0]
    if tuple(alpha.shape) != (D,):
        raise ValueError("alpha must be [D]")
    return D, _shape_arr(grid)


def ecc_height(grid, dirs, alpha, out=None):
    """Heights grid + alpha[d] * <dirs[d], p>: float32[D, *grid.shape] (see include/ecc.h)."""
    D, shp = _height_args(grid, dirs, alpha)
    if out is None:
        out = torch.empty((D,) + tuple(grid.shape), dtype=torch.float32, device=grid.device)
    _dev_tensor(out, "out", torch.float32, grid.device)
    if tuple(out.shape) != (D,) + tuple(grid.shape):
        raise ValueError("out must be [D, *grid.shape]")
    s = _stream(grid)
    check(lib.ecc_height(_ptr(grid), grid.dim(), ctypes.cast(shp, ctypes.c_void_p), _ptr(dirs), _ptr(alpha), D,
                         _ptr(out), s.cuda_stream), "ecc_height")
    return out


def ecc_height_bwd(grad_h, dirs, alpha, need_grid=True, need_dirs=True):
    """(dL/dgrid, dL/ddirs, dL/dalpha) from dL/dheights [D, *shape]; None where not needed."""
    _dev_tensor(grad_h, "grad_h", torch.float32)
    if grad_h.dim() not in (3, 4):
        raise ValueError("grad_h must be [D, *grid.shape]")
    _dev_tensor(dirs, "dirs", torch.float32, grad_h.device)
    _dev_tensor(alpha, "alpha", torch.float32, grad_h.device)
    D, nd = grad_h.shape[0], grad_h.dim() - 1
    if tuple(dirs.shape) != (D, nd) or tuple(alpha.shape) != (D,):
        raise ValueError("dirs must be [D, ndim] and alpha [D]")
    shp = (ctypes.c_int64 * nd)(*grad_h.shape[1:])
    dev = grad_h.device
    gg = torch.empty(tuple(grad_h.shape[1:]), dtype=torch.float32, device=dev) if need_grid else None
    gd = torch.empty((D, nd), dtype=torch.float32, device=dev) if need_dirs else None
    ga = torch.empty((D,), dtype=torch.float32, device=dev) if need_dirs else None
    s = _stream(grad_h)
    nb = int(lib.ecc_height_workspace_bytes(nd, D))
    ws = get_workspace(nb, dev, s)
    null = ctypes.c_void_p(0)
    check(lib.ecc_height_bwd(_ptr(grad_h), nd, ctypes.cast(shp, ctypes.c_void_p), _ptr(dirs), _ptr(alpha), D,
                             _ptr(gg) if gg is not None else null, _ptr(gd) if gd is not None else null,
                             _ptr(ga) if ga is not None else null, _ptr(ws), ws.numel() * ws.element_size(),
                             s.cuda_stream), "ecc_height_bwd")
    return gg, gd, ga


class Heights(torch.autograd.Function):
    """Directional heights as an autograd op: (grid, dirs [D, nd], alpha [D]) -> [D, *grid.shape]."""

    @staticmethod
    def forward(ctx, grid, dirs, alpha):
        ctx.save_for_backward(dirs, alpha)
        return ecc_height(grid.detach().contiguous(), dirs.detach().contiguous(), alpha.detach().contiguous())

    @staticmethod
    def backward(ctx, grad_h):
        dirs, alpha = ctx.saved_tensors
        need_dirs = ctx.needs_input_grad[1] or ctx.needs_input_grad[2]
        gg, gd, ga = ecc_height_bwd(grad_h.contiguous(), dirs.detach().contiguous(), alpha.detach().contiguous(),
                                    need_grid=ctx.needs_input_grad[0], need_dirs=need_dirs)
        return gg, gd if ctx.needs_input_grad[1] else None, ga if ctx.needs_input_grad[2] else None


def directional_heights(grid, dirs, alpha):
    """Heights f[d] = grid + alpha[d] <dirs[d], p>, differentiable in all three inputs."""
    return Heights.apply(grid, dirs, alpha)


def ecc_hard_directional(grid, dirs, alpha, tau):
    """Hard curves of the D directional height grids: int64[D, H]."""
    return ecc_hard_batched(ecc_height(grid, dirs, alpha), tau)


def soft_ecc_directional(grid, dirs, alpha, tau, lam):
    """Soft curves of the D directional height grids, float32[D, H], differentiable
    in the grid, the directions, the scales and the thresholds."""
    return soft_ecc_batched(directional_heights(grid, dirs, alpha), tau, lam)
