"""Compile the HIP sources into exact_lloyd_means_03_amd/libkmeans_mi355x.so (gfx950).

hipcc cross-compiles for gfx950 on a machine without a GPU.  Objects go to
exact_lloyd_means_03_amd/_build/; the shared library is written next to
this file so that it travels with the source tree.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ARCH = os.environ.get("KM_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# KM_SANITIZE=1: the host code (argument checks, workspace plans, launch
# sequences) is built with AddressSanitizer and UndefinedBehaviorSanitizer,
# into _build_san/ next to this file (never over the product library); the
# tests load it when KM_LIBRARY names it (tests/run_sanitized.py does both).
# Device code is built as usual.
SANITIZE = os.environ.get("KM_SANITIZE", "") == "1"
BUILD = os.path.join(HERE, "_build_san" if SANITIZE else "_build")
LIB = os.path.join(BUILD, "libkmeans_mi355x.so") if SANITIZE else os.path.join(HERE, "libkmeans_mi355x.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]

SOURCES = ["small.hip", "assign_mfma.hip", "assign_1d.hip", "fit_1d.hip", "optimal_1d.hip", "emeans.hip",
           "sort.hip", "update.hip", "api.hip"]

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in VGPRs: the epilogue reads them without AGPR copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-fvisibility=hidden",
]

# Per-source extra flags.  The assignment kernel never sees a NaN (inputs are
# finite, padding rows are -inf), so fmaxf needs no NaN canonicalization.
EXTRA = {"assign_mfma.hip": ["-fno-honor-nans"]}


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), *(SAN_FLAGS if SANITIZE else []), "-c", os.path.join(CSRC, src),
           "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *(SAN_FLAGS if SANITIZE else []), *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
