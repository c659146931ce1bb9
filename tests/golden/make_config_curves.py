"""Write tests/golden/config_curves.json: the oracle's whole curves for the
three largest workloads, so the GPU tests can compare every output.

    python tests/golden/make_config_curves.py [--workers N] [--only NAME ...]

Only ``oracle/`` computes anything here; ``workloads.py`` draws the inputs.
The grids are split into z-slabs that run in parallel worker processes and
are added up by inclusion-exclusion (tests/slabs.py, checked against the
whole-grid oracle on small grids by tests/test_golden_config_curves.py).

Recorded per workload: shape, dtype, H, the SHA-256 of the grid's and the
thresholds' bytes (the GPU tests regenerate the inputs and compare these
first), and
  * hard workloads: the int64 curve ``ecc`` (oracle.ecc_hard);
  * the soft workload: ``soft`` (oracle.ecc_soft) and ``soft_bwd_unit``
    (oracle.ecc_soft_bwd_tau with an upstream gradient of ones, i.e.
    lambda * sum_c sign_c sigma sigma'); the backward for an upstream
    gradient g is g_k times entry k, since the threshold Jacobian is diagonal.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from euler_characteristic_curves_amd import workloads as W  # noqa: E402
from tests import slabs  # noqa: E402

OUT = os.path.join(HERE, "config_curves.json")
NAMES = ("c4a_512cube_f32_grf", "c4b_1024cube_f32", "c5_256cube_soft")


def sha256(a):
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8).ravel()).hexdigest()


def record(name, workers):
    g, tau, extra = W.make_workload(name)
    rec = {"shape": list(g.shape), "dtype": str(g.dtype), "H": int(tau.size),
           "grid_sha256": sha256(g), "tau_sha256": sha256(tau)}
    t0 = time.perf_counter()
    if name.startswith("c5"):
        lam = float(extra["lam"])
        rec["lam"] = lam
        rec["soft"] = slabs.curve_combined("soft", g, tau, lam, slab=16, workers=workers).tolist()
        rec["soft_bwd_unit"] = slabs.curve_combined("bwd", g, tau, lam, slab=16, workers=workers).tolist()
    else:
        slab = 32 if g.shape[0] <= 512 else 16
        rec["ecc"] = [int(v) for v in slabs.curve_combined("hard", g, tau, slab=slab, workers=workers)]
    print(f"{name}: {time.perf_counter() - t0:.1f} s", flush=True)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workers", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--only", nargs="*", default=list(NAMES))
    a = ap.parse_args()
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    data.setdefault("about", "Whole oracle curves of the 512^3, 1024^3 and 256^3 soft workloads, "
                             "written by tests/golden/make_config_curves.py from oracle/ only.")
    for name in a.only:
        data[name] = record(name, a.workers)
        with open(OUT, "w") as f:
            json.dump(data, f, indent=0)
            f.write("\n")


if __name__ == "__main__":
    main()
