"""Build libmoeperm.so (HIP, gfx950) in-tree: unpermute_combine_moe_amd/libmoeperm.so.

Every csrc/*.hip file is compiled by hipcc for gfx950 only and linked into one
shared library exporting the C ABI of include/libmoeperm.h.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "libmoeperm")
LIB = os.path.join(PKG, "libmoeperm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep hipcc from forming v_pk_{add,mul,fma}_f32 (the host
# pass warns that it does not know the feature; that is expected).
CXXFLAGS = [
    "-std=c++17", "-O3", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wextra", "-Wno-unused-parameter", "-I" + INCLUDE, "-I" + CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CXXFLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    build_probes(verbose)
    return LIB


def build_probes(verbose: bool = False) -> list:
    """Compile the measurement aids under probes/ (stand-alone executables,
    not part of the library) into _build/probes/, so that they keep building."""
    out_dir = os.path.join(ROOT, "_build", "probes")
    os.makedirs(out_dir, exist_ok=True)
    outs = []
    for src in sorted(glob.glob(os.path.join(PKG, "probes", "*.hip"))):
        exe = os.path.join(out_dir, os.path.splitext(os.path.basename(src))[0])
        cmd = [HIPCC, "-std=c++17", "-O3", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", src, "-o", exe]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}{r.stderr}")
        outs.append(exe)
    return outs


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
