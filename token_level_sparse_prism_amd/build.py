"""Build the gfx950 HIP library libprism.so in-tree (token_level_sparse_prism_amd/lib/).

Every .hip file under csrc/ is compiled with hipcc for gfx950 (in parallel), then linked into
one shared library exporting the C ABI of include/prism.h.

Usage: python -m token_level_sparse_prism_amd.build   (or python token_level_sparse_prism_amd/build.py)
       python -m token_level_sparse_prism_amd.build --timeline
           also builds lib/libprism_tl.so: the same sources with PRISM_TIMELINE=1, whose kernels
           record per-workgroup phase timestamps (a diagnostics build; bench.py --timeline loads it)
       python -m token_level_sparse_prism_amd.build --only-timeline --define NAME=VALUE ... --out FILE
           builds only a timeline library, with extra build settings (for example
           PRISM_SELECT_LEAN=0, the general selection path), as lib/FILE (bench.py --lib loads it)
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libprism.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops are disabled (-packed-fp32-ops): the compiler emits ordinary fp32 ops only.
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


LIB_TL = os.path.join(LIBDIR, "libprism_tl.so")
BUILD_TL = os.path.join(PKG, "_build_tl")


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 0, timeline: bool = False, defines=(), out: str = "") -> str:
    build_dir, lib = (BUILD_TL, LIB_TL) if timeline else (BUILD, LIB)
    if out:
        lib = os.path.join(LIBDIR, os.path.basename(out))
        build_dir = os.path.join(PKG, "_build_" + os.path.splitext(os.path.basename(out))[0])
    extra = (("-DPRISM_TIMELINE=1",) if timeline else ()) + tuple(f"-D{d}" for d in defines)
    os.makedirs(build_dir, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), srcs))
    LIBX = lib
    tmp = LIBX + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIBX)
    if verbose:
        print(f"built {LIBX}", flush=True)
    return LIBX


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--timeline", action="store_true")
    ap.add_argument("--only-timeline", action="store_true")
    ap.add_argument("--define", action="append", default=[])
    ap.add_argument("--out", default="")
    opts = ap.parse_args()
    if not opts.only_timeline:
        build(verbose=True)
    if opts.timeline or opts.only_timeline:
        build(verbose=True, timeline=True, defines=opts.define, out=opts.out)
    sys.exit(0)
