"""Build the C-ABI library from csrc/*.hip for gfx950 with hipcc, in two
variants next to this file:

  libgdn.so       the library (include/gdn.h)
  libgdn_prof.so  the same sources with GDN_PROFILE defined: it also exports the
                  launch recorder of include/gdn_profile.h, for measurement tools

Each .hip file is compiled to an object in parallel (both variants at once),
then each variant is linked into one shared library.
Usage: python -m gated_delta_rule_52_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgdn.so")
LIB_PROF = os.path.join(HERE, "libgdn_prof.so")
VARIANTS = ((LIB, "lib", []), (LIB_PROF, "prof", ["-DGDN_PROFILE"]))
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed-fp32 VALU forms are kept off: plain fp32 ops only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, sub: str, defs: list, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, sub, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *defs, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
    return obj


def _link(objs: list, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every csrc/*.hip and link libgdn.so and libgdn_prof.so; always
    rebuilds.  Returns the path of libgdn.so."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    work = [(s, sub, defs) for _, sub, defs in VARIANTS for s in srcs]
    for _, sub, _ in VARIANTS:
        os.makedirs(os.path.join(OBJDIR, sub), exist_ok=True)
    jobs = jobs or min(len(work), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda w: _compile(*w, verbose), work))
    for i, (lib, _, _) in enumerate(VARIANTS):
        _link(objs[i * len(srcs):(i + 1) * len(srcs)], lib, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
