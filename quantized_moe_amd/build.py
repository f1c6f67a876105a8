"""Build libqmoe.so (the HIP library) in-tree for gfx950.

Each .hip source is compiled separately (the router file with floating-point
contraction off, so its fixed summation order is exactly what the source
says), then linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libqmoe.so")
PROBE_OUT = os.path.join(HERE, "libqmoe_probe.so")  # measurement probes (not the layer's ABI)
OBJ = os.path.join(HERE, "_build")
ARCH = "gfx950"

SOURCES = ["api.hip", "route.hip", "bucket.hip", "repack.hip", "decode.hip", "decode_k1.hip", "decode_k2.hip",
           "decode_k3.hip", "decode_unique.hip", "prefill.hip", "dense.hip"]
PROBE_SOURCES = ["probe.hip"]
# packed-fp32 VALU forms are disabled: only ordinary fp32 instructions
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]
PER_FILE = {"route.hip": ["-ffp-contract=off"]}
# hipBLASLt runs the dense shared-expert GEMMs of long prefill chunks (dense.hip)
LIBS = ["-L/opt/rocm/lib", "-lhipblaslt"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, src.replace(".hip", ".o"))
    cmd = ["hipcc", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + PER_FILE.get(src, [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "hip-link" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs:
        print(msgs, file=sys.stderr)
    return obj


def _link(objs, out, libs=()):
    tmp = out + ".tmp"
    cmd = ["hipcc", "-shared", "-o", tmp, f"--offload-arch={ARCH}"] + objs + list(libs)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(10, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], OUT, LIBS)
    _link(objs[len(SOURCES):], PROBE_OUT)
    if verbose:
        print(f"built {OUT} and {PROBE_OUT}")
    return OUT


if __name__ == "__main__":
    build()
