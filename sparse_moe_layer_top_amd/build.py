"""Build libbeam_moe.so (HIP kernels + C ABI) in-tree for gfx950.

    python sparse_moe_layer_top_amd/build.py

Every .hip file under csrc/ is compiled to an object in _build/ (in parallel),
then linked into sparse_moe_layer_top_amd/libbeam_moe.so.  The compiler's
per-kernel resource report is checked on the way: a kernel that spills
registers or uses scratch memory fails the build.
"""
from __future__ import annotations

import glob
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbeam_moe.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every float multiply and add rounds on its own (the oracle's arithmetic);
    # fused multiply-adds only where the source writes fmaf
    "-ffp-contract=off",
    "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


# the compiler's per-kernel resource report (registers, scratch, spills), checked after each compile
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                     r"SGPRs Spill|VGPRs Spill): (\S+)")


def kernel_resources(remarks: str) -> list:
    """One dict per kernel from the compiler's resource remarks: name, VGPRs, AGPRs, scratch bytes per
    lane, occupancy, SGPR and VGPR spills."""
    out = []
    for line in remarks.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            out.append({"kernel": val})
        elif out:
            out[-1][key.split(" [")[0]] = int(val) if val.lstrip("-").isdigit() else val
    return out


def spilling(kernels: list) -> list:
    """Kernels that use scratch memory or spill registers (each such access is a round trip to memory)."""
    return [k for k in kernels
            if k.get("ScratchSize", 0) != 0 or k.get("VGPRs Spill", 0) != 0 or k.get("SGPRs Spill", 0) != 0]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, RESOURCE_REMARKS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    bad = spilling(kernel_resources(r.stderr))
    if bad:
        raise RuntimeError(f"kernels in {src} spill registers or use scratch memory: {bad}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
