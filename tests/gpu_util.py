"""Helpers for the GPU parity tests: device checks, tolerance, case banners."""

import sys

import numpy as np
import pytest


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    return torch


def banner(*parts):
    """Name the case on stdout before the GPU step (flushed)."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def soft_close(got, ref):
    """Soft ECC tolerance: 1e-4 relative where |ref| >= 10, else 1e-3 absolute."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    tol = np.where(np.abs(ref) >= 10.0, 1e-4 * np.abs(ref), 1e-3)
    err = np.abs(got - ref)
    bad = np.nonzero(~(err <= tol))[0]
    return bad, float(np.max(err / tol)) if err.size else 0.0
