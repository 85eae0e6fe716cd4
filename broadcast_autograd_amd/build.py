"""Builds libzk.so (the gfx950 HIP library behind include/zk.h) in-tree.

    python -m broadcast_autograd_amd.build

Every source is compiled with hipcc for gfx950 only.  Device code keeps IEEE
binary32 semantics: no contraction into FMA (-ffp-contract=off), correctly
rounded division and square root, subnormals kept (no flush flag), and the
packed-FP32 instructions turned off.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libzk.so")

SOURCES = ["zk_plan.cpp", "zk_api.cpp", "zk_fwd.hip", "zk_bwd.hip", "zk_norm.hip",
           "zk_rows.hip", "zk_scratch.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
          "-Wno-uninitialized", "-Wno-unused-command-line-argument",
          "-I", INCLUDE, "-I", CSRC]
DEVICE = ["-x", "hip", "--offload-arch=gfx950", "-ffp-contract=off",
          "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    flags = COMMON + (DEVICE if src.endswith(".hip") else [])
    cmd = [HIPCC] + flags + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
