"""Build the native libraries in-tree for gfx950.

* ``shared_paged_kv_amd/libkvpool.so``: the C-ABI library (host control plane
  compiled with g++, HIP kernels with hipcc).
* ``workload/libkvgen.so``: the seeded input filler used by tests and the bench, and
  the plain read probe the bench measures the read ceiling with.
* ``shared_paged_kv_amd/libkvpool_checked.so``: the same library with the
  kernels' bounds checks on table indices compiled in (``KVP_DEVICE_CHECKS``;
  load it with ``KVPOOL_LIB``, as tests/test_gpu_device_checks.py does).
* on request (``--host-sanitized``), ``_build/san/libkvpool.so``: the same library
  with its host control plane (tables, lifecycle, persistence) built with
  AddressSanitizer and UndefinedBehaviorSanitizer, linked against the ordinary
  HIP objects; load it with ``KVPOOL_LIB`` and the sanitizer runtimes preloaded
  (tests/test_host_sanitized.py does).

Run ``python -m shared_paged_kv_amd.build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

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
# host-only sanitizer flags (g++ lines only; no device code is built with them)
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
HOST_SOURCES = ["tables.cpp", "lifecycle.cpp", "persist.cpp"]
HIP_SOURCES = ["rerotate.hip", "decode.hip", "append.hip", "mirror.hip", "persist.hip"]
BUILD_JOBS = max(1, min(4, os.cpu_count() or 1))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return r


def build_kvpool(verbose: bool = False) -> str:
    """libkvpool.so and libkvpool_checked.so; the compiles run side by side (at
    most BUILD_JOBS at a time, the heavy decode.hip ones first)."""
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(CSRC, "host")]
    jobs, objs = [], []
    dec_checked = os.path.join(BUILD, "decode_checked.hip.o")
    jobs.append([HIPCC, *HIP_FLAGS, "-DKVP_DEVICE_CHECKS", *inc, "-c", os.path.join(CSRC, "hip", "decode.hip"), "-o",
                 dec_checked])
    for f in HIP_SOURCES:
        o = os.path.join(BUILD, f + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "hip", f), "-o", o])
        objs.append(o)
    for f in HOST_SOURCES:
        o = os.path.join(BUILD, f + ".o")
        jobs.append(["g++", *CXX_FLAGS, *inc, "-c", os.path.join(CSRC, "host", f), "-o", o])
        objs.append(o)
    jobs.sort(key=lambda c: "decode.hip" not in " ".join(c))
    with ThreadPoolExecutor(max_workers=BUILD_JOBS) as ex:
        list(ex.map(_run, jobs))
    out = os.path.join(PKG, "libkvpool.so")
    # the checked build: decode.hip with its bounds checks, the other objects as above
    chk = os.path.join(PKG, "libkvpool_checked.so")
    for lib_out, lib_objs in ((out, objs), (chk, [dec_checked if o.endswith(os.sep + "decode.hip.o") else o
                                                  for o in objs])):
        tmp = lib_out + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *lib_objs])
        os.replace(tmp, lib_out)
        if verbose:
            print("built", lib_out)
    return out


def build_host_sanitized(verbose: bool = False) -> str:
    """_build/san/libkvpool.so: host control plane under ASan + UBSan, HIP objects
    as in the ordinary build (rebuilt when missing or older than their source),
    linked with g++."""
    san = os.path.join(BUILD, "san")
    os.makedirs(san, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(CSRC, "host")]
    objs = []
    for f in HOST_SOURCES:
        o = os.path.join(san, f + ".o")
        _run(["g++", "-O1", "-fPIC", "-std=c++17", *SAN_FLAGS, *inc, "-c", os.path.join(CSRC, "host", f), "-o", o])
        objs.append(o)
    for f in HIP_SOURCES:
        o, src = os.path.join(BUILD, f + ".o"), os.path.join(CSRC, "hip", f)
        if not os.path.exists(o) or os.path.getmtime(o) < os.path.getmtime(src):
            _run([HIPCC, *HIP_FLAGS, *inc, "-c", src, "-o", o])
        objs.append(o)
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "lib")
    out = os.path.join(san, "libkvpool.so")
    _run(["g++", "-shared", *SAN_FLAGS, "-o", out, *objs, f"-L{rocm_lib}", "-lamdhip64", f"-Wl,-rpath,{rocm_lib}"])
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
    if "--host-sanitized" in sys.argv[1:]:
        build_host_sanitized(verbose=True)
    else:
        build_all(verbose=True)
