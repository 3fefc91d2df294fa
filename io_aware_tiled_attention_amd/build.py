"""Build libfa_gfx950.so from the HIP sources with hipcc (gfx950 only).

    python -m io_aware_tiled_attention_amd.build [--jobs N] [--save-temps DIR]

Always recompiles.  The library lands next to this file, where the ctypes
binding loads it from.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfa_gfx950.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# measurement library (not the attention path): the register-only MFMA rate
PROBE_NAME = "libfa_probe_gfx950.so"
PROBE_PATH = os.path.join(PKG, PROBE_NAME)
PROBE_SOURCES = ["mfma_peak.hip"]
SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip", "fa_fwd_fp8.hip", "fa_noalloc.hip", "fa_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: a ROCm toolchain is required to build the library")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # no packed fp32 VALU forms anywhere in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]


def build(jobs: int = 4, save_temps: str | None = None, verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(save_temps or objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *common_flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            cmd.append("-save-temps=obj")   # keeps the AMD assembly (.s) beside the object
        res = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))
    link(cc, objs[:len(SOURCES)], LIB_PATH)
    link(cc, objs[len(SOURCES):], PROBE_PATH)
    return LIB_PATH


def link(cc: str, objs, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, path)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--save-temps", default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    path = build(args.jobs, args.save_temps, args.verbose)
    print(path)


if __name__ == "__main__":
    main()
