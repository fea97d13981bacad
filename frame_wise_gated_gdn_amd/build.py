"""Build the HIP library ``libgdn.so`` (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = [os.path.join(CSRC, "gdn_api.cpp"), os.path.join(CSRC, "gdn_kernels.hip"),
           os.path.join(CSRC, "gdn_gram.hip"), os.path.join(CSRC, "gdn_backward.hip"),
           os.path.join(CSRC, "gdn_tconv.hip"), os.path.join(CSRC, "gdn_attn.hip"),
           os.path.join(CSRC, "gdn_fused.hip")]
DEV_HEADERS = [os.path.join(CSRC, "gdn_device.h")]
HEADERS = [os.path.join(ROOT, "include", "gdn.h"), os.path.join(CSRC, "gdn_internal.h"), *DEV_HEADERS]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
OBJ_DIR = os.path.join(PKG, "_build")


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the library."""
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, *inc, "-c", src, "-o", obj]
        return cmd, subprocess.run(cmd, capture_output=True, text=True), obj

    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for cmd, r, _ in results:
        if verbose or r.returncode != 0:
            sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
    if any(r.returncode != 0 for _, r, _ in results):
        raise RuntimeError("hipcc failed building libgdn.so")
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, _, o in results], "-o", LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed linking libgdn.so")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
