"""Build the HIP libraries in-tree for gfx950: ``libkmeans_mi355x.so`` (the
assignment path) and ``libkmeans_mfma_stream.so`` (the MFMA-rate probe that
bench.py reads the assign kernel's rate against).

Run as ``python -m means_nearest_centroid_amd.build``.  hipcc cross-compiles
without a GPU present.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libkmeans_mi355x.so")
SOURCES = [os.path.join(CSRC, f) for f in ("kmeans_kernels.hip", "kmeans_update.hip",
                                           "kmeans_api.hip")]
PROBE_LIBRARY = os.path.join(PKG, "libkmeans_mfma_stream.so")
PROBE_SOURCES = [os.path.join(CSRC, "mfma_stream.hip")]
ARCH = "gfx950"

# Packed-fp32 VALU forms are switched off for all device code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    path = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; set HIPCC")
    return path


def _compile(sources, output, verbose, extra_flags):
    tmp = output + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in res.stderr.splitlines()
            if "packed-fp32-ops" not in ln]   # host pass does not know the feature
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)
    os.replace(tmp, output)
    return output


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile both libraries; returns the assignment library's path."""
    _compile(PROBE_SOURCES, PROBE_LIBRARY, verbose, extra_flags)
    return _compile(SOURCES, LIBRARY, verbose, extra_flags)


if __name__ == "__main__":
    print(build(verbose=True))
