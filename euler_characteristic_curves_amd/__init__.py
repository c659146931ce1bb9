"""Euler characteristic curves of dense 2D/3D grids on AMD Instinct MI355X.

The compute path is libecc_mi355.so (hand-written HIP for gfx950, C ABI in
include/ecc.h); ``euler_characteristic_curves_amd.ecc`` is its thin PyTorch
binding.  The binding is imported lazily so that ``workloads`` (seeded
synthetic inputs) can be used without the built library; any attempt to use
an ECC entry point without the library raises ImportError.
"""

__version__ = "0.1.0"

_API = (
    "ecc_hard_2d", "ecc_hard_3d", "ecc_hard_3d_static", "ecc_hard", "ecc_hard_batched", "ecc_soft_fwd", "ecc_soft_bwd_tau",
    "ecc_soft_bwd_grid", "ecc_soft_fwd_batched", "ecc_soft_bwd_tau_batched", "ecc_soft_bwd_tau_shared",
    "ecc_soft_bwd_grid_batched",
    "workspace_bytes", "workspace_bytes_batched", "get_workspace", "EccError", "SoftECC", "soft_ecc",
    "SoftECCBatched", "soft_ecc_batched", "ecc_height", "ecc_height_bwd", "Heights", "directional_heights",
    "ecc_hard_directional", "soft_ecc_directional",
)

__all__ = list(_API)


def __getattr__(name):
    if name in _API:
        from . import ecc as _ecc
        return getattr(_ecc, name)
    raise AttributeError(name)
