"""Build the C-ABI shared library libultragen.so in-tree for gfx950.

    python -m diffusion_transformer_sparse_amd.build

Compiles csrc/plan.cpp (host) and the gfx950 device code (csrc/kernels.hip:
layout, RoPE and attention forward; csrc/attn_bwd.hip: attention backward;
csrc/warm_start.hip: the warm-start latent)
with hipcc and links them into diffusion_transformer_sparse_amd/libultragen.so.
All device code is built with packed-fp32 instructions disabled.

The same sources built with -DUG_BOUNDS_CHECK give libultragen_debug.so, the
debug build whose kernels record failed index checks in a device word
(ug_debug_bounds_fwd / _bwd / _warm) instead of trapping.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libultragen.so")
DEBUG_OUT = os.path.join(HERE, "libultragen_debug.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I" + os.path.join(ROOT, "include"), "-I/opt/rocm/include"]
DEVICE_SOURCES = ("kernels.hip", "attn_bwd.hip", "warm_start.hip")
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def _build_one(out: str, build_dir: str, defines, verbose: bool) -> str:
    os.makedirs(build_dir, exist_ok=True)
    plan_o = os.path.join(build_dir, "plan.o")
    _run([HIPCC, *COMMON, *defines, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, "plan.cpp"),
          "-o", plan_o], verbose)
    objs = [plan_o]
    for src in DEVICE_SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        _run([HIPCC, *COMMON, *defines, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, debug: bool = True) -> str:
    """Build libultragen.so, and (debug=True) the bounds-checking libultragen_debug.so."""
    _build_one(OUT, BUILD_DIR, [], verbose)
    if debug:
        _build_one(DEBUG_OUT, os.path.join(BUILD_DIR, "debug"), ["-DUG_BOUNDS_CHECK"], verbose)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
