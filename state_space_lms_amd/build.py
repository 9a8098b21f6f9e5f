"""Build librom.so (the gfx950 HIP library behind include/rom.h) in-tree with hipcc.

    python -m state_space_lms_amd.build          # or: from state_space_lms_amd.build import build; build()

Every source is compiled for gfx950 only, with packed-fp32 instruction selection turned off
(-packed-fp32-ops), then linked into state_space_lms_amd/_lib/librom.so. Only the rom_* symbols
of the C ABI are exported.
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
OUT_DIR = os.path.join(PKG, "_lib")
LIBRARY = os.path.join(OUT_DIR, "librom.so")
SOURCES = ["rom_api.hip", "rom_route.hip", "rom_gemm.hip", "rom_gemv.hip", "rom_conv.hip", "rom_bwd.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build librom")


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    cc = hipcc()
    objs = []

    def compile_one(src):
        obj = os.path.join(OUT_DIR, src.replace(".hip", ".o"))
        cmd = [cc, *FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        # the host pass does not know the gfx950-only feature flag; that warning is expected
        noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
        msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIBRARY)
    for o in objs:
        os.remove(o)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
