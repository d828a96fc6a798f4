"""Build the FwPKM C-ABI shared library for gfx950 with hipcc (in-tree).

    python -m sparse_weight_memory_amd.build            # -> sparse_weight_memory_amd/libfwpkm.so
    python -m sparse_weight_memory_amd.build --checked  # -> libfwpkm_checked.so (device checks)
    python -m sparse_weight_memory_amd.build --debug    # -O0 -g host and device code

Every source is compiled as HIP for gfx950 only; packed-fp32 instructions are
kept out of the device code.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfwpkm.so")
CHECKED_LIB = os.path.join(PKG, "libfwpkm_checked.so")

SOURCES = ["ka_score.hip", "kb_read.hip", "kc_sort.hip", "kd_update.hip", "ke_addr.hip",
           "kf_sequence.hip", "fwpkm_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags(debug: bool = False, checked: bool = False) -> list:
    flags = [
        f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-Wall",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]
    flags += ["-O0", "-g"] if debug else ["-O3"]
    if checked:
        flags += ["-DFWPKM_DEVICE_CHECKS=1"]
    return flags


def build(verbose: bool = False, debug: bool = False, checked: bool = False) -> str:
    """Compile every source and link the library; returns its path.  checked:
    the build with device-side invariant tests, written to CHECKED_LIB (its
    objects in _build/checked) so that the product library stays as it is."""
    out_dir = os.path.join(BUILD, "checked") if checked else BUILD
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    flags = common_flags(debug, checked)

    def compile_one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, "-x", "hip", *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{out}")
        if verbose and out.strip():
            print(out)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = CHECKED_LIB if checked else LIB
    tmp = lib + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv, debug="--debug" in sys.argv, checked="--checked" in sys.argv)
    print(path)
