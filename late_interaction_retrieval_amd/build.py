"""Compile libmaxsim.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m late_interaction_retrieval_amd.build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmaxsim.so")
SOURCES = ["fwd.hip", "bwd.hip", "topk.hip", "ooc.hip", "chamfer.hip", "noalloc.hip", "capi.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # fp32 products and sums are separate IEEE operations unless fmaf is asked for
    "-ffp-contract=off",
    # inputs are finite: max needs no NaN canonicalisation (infinities are kept)
    "-fno-honor-nans",
    # no packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(sources, lib, verbose, extra):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra) + [
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ] + [os.path.join(CSRC, s) for s in sources] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, lib)
    return lib


def build(verbose=False, extra=()):
    """Build libmaxsim.so."""
    return _compile(SOURCES, LIB, verbose, extra)


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
    print(LIB)
