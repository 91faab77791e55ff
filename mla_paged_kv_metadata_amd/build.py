"""Build libmla.so (HIP C++ for gfx950) in-tree with hipcc.

    python -m mla_paged_kv_metadata_amd.build

Each source is compiled to an object in csrc/_build/ (in parallel), then
linked into mla_paged_kv_metadata_amd/libmla.so; the benchmark's
read-bandwidth reference goes into libmla_bw.so.  No GPU is needed to build.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(CSRC, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmla.so")
# The benchmark's read-bandwidth reference (not part of the decode ABI).
LIB_BW = os.path.join(HERE, "libmla_bw.so")
BW_SOURCE = "hbm_read.hip"
ARCH = os.environ.get("MLA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["mla_api.cpp", "mla_metadata.hip", "mla_decode.hip", "mla_decode_narrow.hip",
           "mla_decode_wide.hip", "mla_append.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # hipcc must not form packed fp32 arithmetic on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str, extra, objdir: str = BUILD) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc(), *COMMON, *extra, "-c", *lang, os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra=None, verbose: bool = False, out: str = LIB, objdir: str = BUILD, link_extra=None) -> str:
    """Compile every HIP source and link libmla.so (or `out`, with objects in
    `objdir`); returns its path."""
    extra = list(extra or [])
    os.makedirs(objdir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, objdir), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *(link_extra or []), *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    if out == LIB:
        build_bw(verbose=verbose)
    return out


def build_bw(verbose: bool = False) -> str:
    """Compile the read-bandwidth reference kernel into libmla_bw.so."""
    os.makedirs(BUILD, exist_ok=True)
    obj = _compile(BW_SOURCE, [], BUILD)
    tmp = LIB_BW + ".tmp"
    r = subprocess.run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_BW)
    if verbose:
        print(f"built {LIB_BW}")
    return LIB_BW


if __name__ == "__main__":
    build(extra=sys.argv[1:], verbose=True)
