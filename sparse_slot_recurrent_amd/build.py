"""Builds libramnet.so (the HIP kernels and the C ABI) for gfx950, in-tree.

hipcc cross-compiles without a GPU.  Packed-fp32 instruction selection is
switched off for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libramnet.so")
# Device peak probes for the benchmark (HBM copy, LDS read), a library of
# their own: they are measurement tools, not part of the C ABI.
PROBE_SRC = "probe.hip"
PROBE_LIB = os.path.join(PKG, "libramnet_probe.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "decode.hip", "scan_serial.hip", "scan_chunked.hip", "scan_ranges.hip",
           "step_fused.hip", "tier.hip", "proj.hip", "backward.hip"]
# hipBLASLt carries the dense projections around the layer.
LIBS = ["-L/opt/rocm/lib", "-lhipblaslt"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the RAM-Net HIP library cannot be built")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + [PROBE_SRC]))
    probe_obj = objs.pop()
    tmp = PROBE_LIB + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, probe_obj],
                   check=True)
    os.replace(tmp, PROBE_LIB)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, *LIBS]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
