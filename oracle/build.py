"""Compile the C oracle (plain Lloyd, fp64) into oracle/liblloyd_oracle.so.

Test infrastructure: the library never loads it.  gcc, -O2, OpenMP, no
floating-point contraction and no fast-math, so the fp64 loops run as written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lloyd_oracle.c")
# KM_SANITIZE=1: built with clang's AddressSanitizer and
# UndefinedBehaviorSanitizer (the runtime the sanitized HIP host code uses)
# into _build_san/; the tests load it when KM_ORACLE_LIBRARY names it.
SANITIZE = os.environ.get("KM_SANITIZE", "") == "1"
LIB = os.path.join(HERE, "_build_san", "liblloyd_oracle.so") if SANITIZE else os.path.join(HERE, "liblloyd_oracle.so")
CLANG = "/opt/rocm/llvm/bin/clang"


def compile_source(src: str, out: str, verbose: bool = False) -> str:
    """Compile an oracle C source into the shared library `out`."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    if SANITIZE and out == LIB:
        cmd = [CLANG, "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
               "-shared", "-fPIC", src, "-o", tmp, "-lm"]
    else:
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall",
               "-shared", "-fPIC", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    return compile_source(SRC, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
