"""Host check of the library's correctly rounded float32 square root
(sparse_moe_layer_top_amd/csrc/rn_math.h), compiled with g++ from the same
header the kernels include, against NumPy's float32 sqrt (IEEE, correctly
rounded) on random and near-midpoint inputs."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "sparse_moe_layer_top_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <vector>
#include "rn_math.h"
int main() {
  std::vector<float> v;
  float x;
  while (fread(&x, 4, 1, stdin) == 1) v.push_back(x);
  for (float& y : v) y = beam::sqrt_rn(y);
  fwrite(v.data(), 4, v.size(), stdout);
  return 0;
}
"""


@pytest.fixture(scope="module")
def sqrt_rn_exe(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("rn")
    src = d / "drv.cpp"
    src.write_text(DRIVER)
    exe = d / "drv"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", HEADER_DIR, str(src), "-o", str(exe)], check=True)
    return str(exe)


def _run(exe, xs):
    xs = np.ascontiguousarray(xs, np.float32)
    out = subprocess.run([exe], input=xs.tobytes(), capture_output=True, check=True).stdout
    return np.frombuffer(out, np.float32)


def test_sqrt_rn_random(sqrt_rn_exe):
    rng = np.random.default_rng(0)
    e = rng.uniform(-120, 120, 500_000)
    xs = (np.exp2(e) * rng.uniform(1, 2, e.size)).astype(np.float32)
    got = _run(sqrt_rn_exe, xs)
    assert np.array_equal(got, np.sqrt(xs))


def test_sqrt_rn_near_midpoints(sqrt_rn_exe):
    # x = fp32(m^2) and its neighbours, m the midpoint between two floats: the
    # cases where a root within an ulp most often rounds the wrong way
    rng = np.random.default_rng(1)
    s = (rng.uniform(0.5, 4.0, 100_000)).astype(np.float32)
    nxt = np.nextafter(s, np.float32(np.inf))
    m = (s.astype(np.float64) + nxt.astype(np.float64)) / 2
    x0 = (m * m).astype(np.float32)
    xs = np.concatenate([x0, np.nextafter(x0, np.float32(0)), np.nextafter(x0, np.float32(np.inf)),
                         (s.astype(np.float64) ** 2).astype(np.float32)])
    got = _run(sqrt_rn_exe, xs)
    assert np.array_equal(got, np.sqrt(xs))


def test_sqrt_rn_exact_squares_and_small(sqrt_rn_exe):
    xs = np.array([1, 2, 4, 0.25, 9, 1e-6, 1e-30, 3.4e38, 1.1754944e-38], np.float32)
    assert np.array_equal(_run(sqrt_rn_exe, xs), np.sqrt(xs))
