"""Builds libgdr2.so (the HIP library behind include/gdr2.h) in-tree for gfx950.

    python -m gated_delta_rule_gdr2_amd.build [--poison-lds --out PATH]

Every source is compiled with hipcc for --offload-arch=gfx950 and packed fp32
arithmetic disabled (-Xclang -target-feature -Xclang -packed-fp32-ops; the host
pass warns that it does not know the feature, which is harmless).

--poison-lds builds the debug variant in which every kernel first fills its LDS with
NaN bytes (GDR2_POISON_LDS), to PATH (not the library the package loads); the test
suite runs against it with GDR2_LIB=PATH.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdr2.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["gdr2_api.cpp", "gdr2_fwd.hip", "gdr2_bwd.hip", "gdr2_chain.hip", "gdr2_step.hip", "gdr2_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, build_dir: str, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-D" + d for d in defines] + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    build_dir = BUILD_DIR if not defines else BUILD_DIR + "_" + "_".join(d.lower() for d in defines)
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines), SOURCES))
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libgdr2.so for gfx950")
    ap.add_argument("--poison-lds", action="store_true", help="debug variant: kernels fill their LDS with NaN first")
    ap.add_argument("--out", default=None, help="output path (required with --poison-lds)")
    args = ap.parse_args()
    if args.poison_lds and (args.out is None or os.path.abspath(args.out) == LIB):
        ap.error("--poison-lds needs --out PATH other than the package's library")
    build(verbose=True, out=args.out or LIB, defines=("GDR2_POISON_LDS",) if args.poison_lds else ())
    sys.exit(0)
