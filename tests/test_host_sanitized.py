"""Host code of the library on the CPU, built with g++ under AddressSanitizer
and UndefinedBehaviorSanitizer (no GPU, no HIP runtime):

* tests/host/abi_contract.cpp drives every C ABI entry point of ecc_api.cpp
  against the stubs of tests/host/hip_stubs.cpp: statuses and messages of
  bad arguments, and the exact arguments each launcher receives;
* tests/host/star_count_check.cpp checks c(p) from neighbour bits
  (ecc_star.hpp) against a cell-by-cell count over every neighbour mask
  (sanitized on a sample, plain -O2 on all 2^26 3D masks).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
CSRC = os.path.join(ROOT, "euler_characteristic_curves_amd", "csrc")
HIP_INC = "/opt/rocm/include"
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
INC = ["-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{HIP_INC}", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


@pytest.fixture(scope="module")
def gxx():
    cxx = shutil.which("g++")
    if cxx is None or not os.path.exists(os.path.join(HIP_INC, "hip", "hip_runtime_api.h")):
        pytest.skip("g++ or the HIP headers are not available")
    return cxx


def _build(cxx, out, sources, flags):
    r = subprocess.run([cxx] + flags + INC + sources + ["-o", out], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def _run(args):
    return subprocess.run(args, capture_output=True, text=True, env=ENV, timeout=300)


def test_sanitizer_is_live(gxx, tmp_path):
    """A heap read past the end is reported, so a clean run below means something."""
    src = tmp_path / "overread.cpp"
    src.write_text("#include <vector>\nint main(int c, char**) { std::vector<long> v(3); return (int)v.data()[c + 2]; }\n")
    exe = _build(gxx, str(tmp_path / "overread"), [str(src)], SAN)
    r = _run([exe])
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_abi_contract_under_sanitizers(gxx, tmp_path):
    exe = _build(gxx, str(tmp_path / "abi_contract"),
                 [os.path.join(CSRC, "ecc_api.cpp"), os.path.join(HOST, "hip_stubs.cpp"),
                  os.path.join(HOST, "abi_contract.cpp")], SAN)
    r = _run([exe])
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


def test_star_count_every_mask(gxx, tmp_path):
    src = [os.path.join(HOST, "star_count_check.cpp")]
    san = _build(gxx, str(tmp_path / "star_san"), src, SAN)
    r = _run([san, "61"])                 # 1.1 M of the 3D masks under the sanitizers
    assert r.returncode == 0, r.stdout + r.stderr
    full = _build(gxx, str(tmp_path / "star_full"), src, ["-O2"])
    r = _run([full])                      # all 2^8 2D and 2^26 3D masks
    assert r.returncode == 0, r.stdout + r.stderr
    assert "67109120 masks, 0 mismatches, 3D c(p) in [-5, 7]" in r.stdout
