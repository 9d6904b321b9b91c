"""Build the HIP library libeqlinear.so for gfx950, in-tree.

    python -m group_circulant_linear_p4_amd.build        # or build_library()

Every source under csrc/ is compiled by hipcc into _build/ (in parallel) and
linked into group_circulant_linear_p4_amd/libeqlinear.so.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libeqlinear.so")
# Debug variant: every LDS ring chunk set to NaN before its DMA load (EQL_POISON_RING);
# load it with EQL_LIBRARY=<this path> to run the tests against it.
POISON_LIB = os.path.join(PKG, "libeqlinear_poison.so")
ARCH = os.environ.get("EQL_OFFLOAD_ARCH", "gfx950")

SOURCES = [
    "eql_api.hip",
    "eql_pack.hip",
    "eql_fwd_f16.hip",
    "eql_fwd_f32.hip",
    "eql_fwd_fused_f16.hip",
    "eql_fwd_fused_f32.hip",
    "eql_fwd_spec.hip",
    "eql_bwdw_f16.hip",
    "eql_bwdw_f32.hip",
    "eql_bwdw_real_f16.hip",
    "eql_bwdw_real_f32.hip",
    "eql_bwdw_pair_f16.hip",
    "eql_bwdw_pair_f32.hip",
    "eql_bwdw4.hip",
    "eql_epi.hip",
    "eql_p4m.hip",
]

CFLAGS = [
    "-O3", "-std=c++20", "-fPIC", "--offload-arch=" + ARCH,
    # No packed-fp32 instructions: every fp32 op is scalar per lane.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Rounding is decided by the source: no implicit multiply-add contraction.
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the EQ-Linear library needs ROCm to build")
    return path


def _compile(src: str, extra: list[str], reuse: bool = False, build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    if reuse and os.path.exists(obj):
        return obj
    cmd = [hipcc(), *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr[-8000:]))
    return obj


def build_library(jobs: int | None = None, extra_flags: list[str] | None = None, verbose: bool = False,
                  only: list[str] | None = None, poison_ring: bool = False) -> str:
    """Compile every source and link libeqlinear.so; returns the library path.

    only: recompile just these sources and reuse the other objects of an earlier full
    build (for iterating on one translation unit; the default compiles everything).
    poison_ring: build the debug variant libeqlinear_poison.so instead (objects in
    _build/poison)."""
    build_dir = os.path.join(BUILD, "poison") if poison_ring else BUILD
    lib = POISON_LIB if poison_ring else LIB
    os.makedirs(build_dir, exist_ok=True)
    extra = list(extra_flags or []) + (["-DEQL_POISON_RING"] if poison_ring else [])
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    unknown = sorted(set(only or ()) - set(SOURCES))
    if unknown:
        raise ValueError("not library sources: %s (sources: %s)" % (", ".join(unknown), ", ".join(SOURCES)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, reuse=only is not None and s not in only,
                                              build_dir=build_dir), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr[-8000:]))
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    # python -m group_circulant_linear_p4_amd.build [--poison-ring] [source.hip ...]: with
    # source arguments, only those are recompiled (see build_library's `only`).
    args = sys.argv[1:]
    poison = "--poison-ring" in args
    names = [a for a in args if a != "--poison-ring"]
    build_library(verbose=True, only=names or None, poison_ring=poison)
    sys.exit(0)
