"""Build the native libraries in-tree for gfx950.

* ``shared_paged_kv_amd/libkvpool.so``: the C-ABI library (host control plane
  compiled with g++, HIP kernels with hipcc).
* ``workload/libkvgen.so``: the seeded input filler used by tests and the bench, and
  the plain read probe the bench measures the read ceiling with.

Run ``python -m shared_paged_kv_amd.build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "shared_paged_kv_amd")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 instructions stay off (hipcc's host pass warns that it does not
    # know the feature; that is harmless)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return r


def build_kvpool(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(CSRC, "host")]
    objs = []
    for f in ["tables.cpp", "lifecycle.cpp", "persist.cpp"]:
        o = os.path.join(BUILD, f + ".o")
        _run(["g++", *CXX_FLAGS, *inc, "-c", os.path.join(CSRC, "host", f), "-o", o])
        objs.append(o)
    for f in ["rerotate.hip", "decode.hip", "append.hip", "mirror.hip", "persist.hip"]:
        o = os.path.join(BUILD, f + ".o")
        _run([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "hip", f), "-o", o])
        objs.append(o)
    out = os.path.join(PKG, "libkvpool.so")
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs])
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


def build_kvgen(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for name in ("kvgen.hip", "readprobe.hip"):
        src = os.path.join(ROOT, "workload", "csrc", name)
        o = os.path.join(BUILD, name + ".o")
        _run([HIPCC, *HIP_FLAGS, "-c", src, "-o", o])
        objs.append(o)
    out = os.path.join(ROOT, "workload", "libkvgen.so")
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs])
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


def build_all(verbose: bool = False):
    return build_kvpool(verbose), build_kvgen(verbose)


if __name__ == "__main__":
    build_all(verbose=True)
