"""ctypes loader for libecc_mi355.so (the C ABI declared in include/ecc.h).

Loading fails loudly: there is no fallback implementation of any operation.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libecc_mi355.so")

# status codes and enums mirrored from include/ecc.h
ECC_OK = 0
ECC_E_NULL = 1
ECC_E_SHAPE = 2
ECC_E_DTYPE = 3
ECC_E_NTHRESH = 4
ECC_E_LAMBDA = 5
ECC_E_WORKSPACE = 6
ECC_E_HIP = 7
ECC_E_NDIRS = 8
ECC_U8 = 0
ECC_F32 = 1
ECC_OP_HARD = 0
ECC_OP_SOFT_FWD = 1
ECC_OP_SOFT_BWD = 2
ECC_MAX_THRESHOLDS = 8192
ECC_MAX_DIRECTIONS = 4096

EXPORTS = (
    "ecc_hard_2d", "ecc_hard_3d", "ecc_hard_3d_static", "ecc_hard_2d_batched", "ecc_hard_3d_batched",
    "ecc_soft_fwd", "ecc_soft_bwd_tau", "ecc_soft_bwd_grid",
    "ecc_soft_fwd_batched", "ecc_soft_bwd_tau_batched", "ecc_soft_bwd_tau_shared", "ecc_soft_bwd_grid_batched",
    "ecc_height", "ecc_height_bwd", "ecc_height_workspace_bytes",
    "ecc_workspace_bytes", "ecc_workspace_bytes_batched", "ecc_status_string", "ecc_last_error", "ecc_version",
)


class EccError(RuntimeError):
    """A libecc_mi355 entry point returned a non-zero status."""

    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m euler_characteristic_curves_amd.build` "
            "(ROCm hipcc, gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    F = ctypes.c_float
    lib.ecc_hard_2d.argtypes = [P, I, I64, I64, P, I32, P, P, SZ, P]
    lib.ecc_hard_2d.restype = I
    lib.ecc_hard_3d.argtypes = [P, I, I64, I64, I64, P, I32, P, P, SZ, P]
    lib.ecc_hard_3d.restype = I
    lib.ecc_hard_3d_static.argtypes = [P, I, I64, I64, I64, P, I32, P, P]
    lib.ecc_hard_3d_static.restype = I
    lib.ecc_hard_2d_batched.argtypes = [P, I, I64, I64, I64, P, I64, I32, P, P, SZ, P]
    lib.ecc_hard_2d_batched.restype = I
    lib.ecc_hard_3d_batched.argtypes = [P, I, I64, I64, I64, I64, P, I64, I32, P, P, SZ, P]
    lib.ecc_hard_3d_batched.restype = I
    lib.ecc_soft_fwd.argtypes = [P, I32, P, P, I32, F, P, P, SZ, P]
    lib.ecc_soft_fwd.restype = I
    lib.ecc_soft_bwd_tau.argtypes = [P, I32, P, P, I32, F, P, P, P, SZ, P]
    lib.ecc_soft_bwd_tau.restype = I
    lib.ecc_soft_bwd_grid.argtypes = [P, I32, P, P, I32, F, P, P, P]
    lib.ecc_soft_bwd_grid.restype = I
    lib.ecc_soft_fwd_batched.argtypes = [P, I32, P, I64, P, I64, I32, F, P, P, SZ, P]
    lib.ecc_soft_fwd_batched.restype = I
    lib.ecc_soft_bwd_tau_batched.argtypes = [P, I32, P, I64, P, I64, I32, F, P, P, P, SZ, P]
    lib.ecc_soft_bwd_tau_batched.restype = I
    lib.ecc_soft_bwd_tau_shared.argtypes = [P, I32, P, I64, P, I32, F, P, P, P, SZ, P]
    lib.ecc_soft_bwd_tau_shared.restype = I
    lib.ecc_soft_bwd_grid_batched.argtypes = [P, I32, P, I64, P, I64, I32, F, P, P, P]
    lib.ecc_soft_bwd_grid_batched.restype = I
    lib.ecc_height.argtypes = [P, I32, P, P, P, I32, P, P]
    lib.ecc_height.restype = I
    lib.ecc_height_bwd.argtypes = [P, I32, P, P, P, I32, P, P, P, P, SZ, P]
    lib.ecc_height_bwd.restype = I
    lib.ecc_height_workspace_bytes.argtypes = [I32, I32]
    lib.ecc_height_workspace_bytes.restype = SZ
    lib.ecc_workspace_bytes.argtypes = [I, I32, P, I32]
    lib.ecc_workspace_bytes.restype = SZ
    lib.ecc_workspace_bytes_batched.argtypes = [I, I64, I32]
    lib.ecc_workspace_bytes_batched.restype = SZ
    lib.ecc_status_string.argtypes = [I]
    lib.ecc_status_string.restype = ctypes.c_char_p
    lib.ecc_last_error.argtypes = []
    lib.ecc_last_error.restype = ctypes.c_char_p
    lib.ecc_version.argtypes = []
    lib.ecc_version.restype = ctypes.c_char_p
    return lib


lib = _load()


def check(status, what):
    if status != ECC_OK:
        detail = lib.ecc_last_error().decode(errors="replace")
        text = lib.ecc_status_string(status).decode(errors="replace")
        raise EccError(status, f"{what}: {text} ({detail})")
