"""Access to tests/golden/config_curves.json (whole oracle curves of the large
workloads, written by tests/golden/make_config_curves.py from oracle/ only)."""

import hashlib
import json
import os

import numpy as np

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "config_curves.json")


def load(name):
    with open(PATH) as f:
        return json.load(f)[name]


def sha256(a):
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8).ravel()).hexdigest()


def same_inputs(rec, grid, tau):
    """True when grid and tau are byte for byte the inputs the record was made from."""
    return (list(grid.shape) == rec["shape"] and str(grid.dtype) == rec["dtype"]
            and sha256(grid) == rec["grid_sha256"] and sha256(tau) == rec["tau_sha256"])
