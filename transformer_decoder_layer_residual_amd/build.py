"""Build libdl_layer.so (HIP, gfx950) in-tree.

Each csrc/*.hip file is compiled to an object in parallel with hipcc and the
objects are linked into transformer_decoder_layer_residual_amd/libdl_layer.so.
The measurement kernels of csrc/probe/ (achievable read, copy and MFMA rates,
used only by the profiling tool) become libdl_probe.so beside it.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "libdl_layer.so")
PROBE_LIB = os.path.join(PKG, "libdl_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("DL_OFFLOAD_ARCH", "gfx950")

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # never emit packed fp32 ALU ops (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link the shared library.  Always rebuilds."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    build_probe(verbose)
    return LIB


def build_probe(verbose: bool = True) -> str:
    """Compile csrc/probe/*.hip into libdl_probe.so (measurement kernels)."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip")))
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *CFLAGS, "-shared", "-o", tmp, *srcs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        err = "\n".join(l for l in (r.stderr or "").splitlines()
                        if "is not a recognized feature for this target" not in l)
        raise RuntimeError("probe library build failed:\n" + err)
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}", file=sys.stderr)
    return PROBE_LIB


if __name__ == "__main__":
    build()
