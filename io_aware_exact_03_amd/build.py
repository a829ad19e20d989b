"""Build libfa.so for gfx950 in-tree: hipcc compiles every csrc/*.hip, links
one shared library next to this file.  Run as ``python -m
io_aware_exact_03_amd.build`` or through ``__graft_entry__.build()``.

``python -m io_aware_exact_03_amd.build --variant NAME -D MACRO=VALUE ...``
builds the same sources with other tile constants (the FA_* defines of
csrc/fa_plan.hpp) into _build/variants/NAME/libfa.so, which the loader takes
from the IO_AWARE_FA_LIB environment variable (bench.py --lib); the shipped
library is left alone."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfa.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(os.path.dirname(HERE), "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, build_dir: str, defines: tuple) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *(f"-D{d}" for d in defines), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def variant_lib(name: str) -> str:
    return os.path.join(BUILD, "variants", name, "libfa.so")


def build(verbose: bool = True, variant: str | None = None, defines: tuple = ()) -> str:
    """Compile and link; returns the library path.  With a variant name the
    defines (MACRO=VALUE strings) apply and the library goes to
    variant_lib(name)."""
    if variant is None and defines:
        raise ValueError("defines need a variant name")
    build_dir = BUILD if variant is None else os.path.dirname(variant_lib(variant))
    lib = LIB if variant is None else variant_lib(variant)
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), max(1, (os.cpu_count() or 2)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, tuple(defines)), srcs))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources" + (f" with {' '.join(defines)}" if defines else ""))
    return lib


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--variant", help="build a tile variant into _build/variants/NAME")
    ap.add_argument("-D", dest="defines", action="append", default=[], metavar="MACRO=VALUE",
                    help="a define for the variant (repeatable)")
    a = ap.parse_args()
    build(variant=a.variant, defines=tuple(a.defines))
    sys.exit(0)
