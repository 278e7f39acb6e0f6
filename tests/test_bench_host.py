"""bench.py's host logic (no GPU): the gate/up kernel family it names for each workload follows the
library's schedule (the kernels the committed rocprofv3 traces show), the traffic figures are read
only for the sources and weight order they were taken with, and --gpus above 1 is refused."""
import json
import os
import subprocess
import sys

import pytest

import bench
from synth import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (workload, weights in fragment order, kernel family); the fragment-order rows are the kernels named
# by the committed profiles of those workloads
SCHEDULES = [
    ("decode", True, "stream"), ("fp8_decode", True, "stream"), ("mxfp4_decode", True, "stream"),
    ("spec_verify", True, "stream"), ("prefill", True, "wide"), ("skew", True, "wide"),
    ("fp8_prefill", True, "wide"), ("mxfp4_prefill", True, "wide"), ("dense_prefill", True, "wide"),
    ("dense_decode", True, "stream"),
    # row order: the 272-row gate/up only from 192 rows per expert, the LDS-tiled kernels below
    ("prefill", False, "wide"), ("skew", False, "tiled"),
]


@pytest.mark.parametrize("name,packed,kind", SCHEDULES)
def test_gateup_kind(name, packed, kind):
    assert bench.gateup_kind(gen.workload(name), packed=packed) == kind


def test_committed_traffic_matches_its_profile():
    for name in ("decode", "prefill", "skew", "fp8_prefill", "mxfp4_prefill"):
        path = os.path.join(ROOT, "profiles", f"gateup_{name}_traffic.json")
        d = json.load(open(path))
        kind = bench.gateup_kind(gen.workload(name), packed=d["weight_order"] == "fragments")
        fam = {"stream": "gateup_stream_kernel", "wide": "wide_kernel", "tiled": "tiled_kernel"}[kind]
        assert fam in d["kernel"], (name, d["kernel"], kind)
        assert os.path.exists(os.path.join(ROOT, d["summary"]))
        # read for the order it was taken with only
        assert bench.load_traffic(name, "gateup", kind, d["weight_order"]) in (None, d["bytes_per_launch"])
        other = "rows" if d["weight_order"] == "fragments" else "fragments"
        assert bench.load_traffic(name, "gateup", kind, other) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
