"""The CPU test tier with the host code under AddressSanitizer and
UndefinedBehaviorSanitizer.

Builds the HIP library's host code (argument checks, workspace plans, the
launch sequences up to the first HIP call) and the C oracle with clang's
ASan + UBSan into their _build_san/ folders, then runs
`pytest -m "not gpu"` with those builds loaded (KM_LIBRARY,
KM_ORACLE_LIBRARY) and the sanitizer runtime preloaded into the Python
process.  Any report fails the run.  The product library is not touched.

    python tests/run_sanitized.py [extra pytest args]
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def main() -> int:
    env = dict(os.environ, KM_SANITIZE="1")
    for script in ("exact_lloyd_means_03_amd/build.py", "oracle/build.py"):
        subprocess.run([sys.executable, os.path.join(ROOT, script)], check=True, env=env, cwd=ROOT)
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        raise SystemExit("clang's ASan runtime was not found under /opt/rocm/llvm")
    run_env = dict(os.environ)
    run_env.pop("KM_SANITIZE", None)
    run_env.update(
        KM_LIBRARY=os.path.join(ROOT, "exact_lloyd_means_03_amd", "_build_san", "libkmeans_mi355x.so"),
        KM_ORACLE_LIBRARY=os.path.join(ROOT, "oracle", "_build_san", "liblloyd_oracle.so"),
        # the sanitizer runtime goes first; whatever the environment already
        # preloads stays loaded after it
        LD_PRELOAD=":".join(x for x in (rt[-1], os.environ.get("LD_PRELOAD", "")) if x),
        # the interpreter and torch keep memory until exit: leaks are not checked
        ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
        UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
    )
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu", "-p",
           "no:cacheprovider", *sys.argv[1:]]
    return subprocess.run(cmd, env=run_env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main())
