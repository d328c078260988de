"""AddressSanitizer + UndefinedBehaviorSanitizer run of the host code (CPU only).

Builds, into tests/sanitize/_build/:
  * the oracle (oracle/kvq_oracle.c) with gcc -fsanitize=address,undefined;
  * the C-ABI library with the sanitizers on its host code only (every
    -fsanitize= goes behind -Xarch_host: the GPU code is built as usual);
then runs CPU test files against those builds, each in its own process with
that sanitizer's runtime preloaded (gcc's for the oracle, clang's for the
library), leak detection off (the Python interpreter itself would report),
and any undefined behaviour made fatal.  Exit status 0 when every run is
clean.  Usage: python tests/sanitize/run_sanitizers.py [--quick]
(--quick runs the oracle tests without the exhaustive sweeps).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BUILD = os.path.join(HERE, "_build")
HIPCC = "/opt/rocm/bin/hipcc"
CSRC = os.path.join(ROOT, "quantized_kv_cache_fp8_amd", "csrc")
SAN = ["address", "undefined"]


def sh(cmd, **kw):
    print("+", " ".join(cmd), flush=True)
    subprocess.check_call(cmd, **kw)


def build_oracle() -> str:
    out = os.path.join(BUILD, "liborc_san.so")
    sh(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-omit-frame-pointer",
        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
        os.path.join(ROOT, "oracle", "kvq_oracle.c"), "-o", out, "-lm"])
    return out


def build_library() -> str:
    host_san = []
    for s in SAN:
        host_san += ["-Xarch_host", f"-fsanitize={s}"]
    host_san += ["-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
                 "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang",
             "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics"]
    objs = []
    procs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        cmd = [HIPCC, *flags, *host_san, "-c", src, "-o", obj]
        print("+", " ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd))
        objs.append(obj)
    for p in procs:
        if p.wait() != 0:
            raise SystemExit("sanitizer build failed")
    out = os.path.join(BUILD, "libkvq_san.so")
    sh([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *host_san, *objs, "-o", out])
    return out


def instrumented(lib: str) -> None:
    """The build really carries both sanitizers' checks."""
    syms = subprocess.check_output(["nm", "-D", "--undefined-only", lib], text=True)
    for tag in ("__asan_report", "__ubsan_handle"):
        if tag not in syms:
            raise SystemExit(f"{lib}: no {tag}* references, the sanitizer build is not instrumented")


def runtime(kind: str) -> str:
    if kind == "gcc":
        return subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    libs = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not libs:
        raise SystemExit("clang's ASan runtime not found")
    return libs[0]


def run_pytest(files, extra_env, preload, deselect=()):
    env = dict(os.environ)
    env.update(extra_env)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:allow_user_segv_handler=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *files]
    for d in deselect:
        cmd += ["-k", d]
    print("+", " ".join(cmd), flush=True)
    return subprocess.call(cmd, cwd=ROOT, env=env)


def main() -> int:
    quick = "--quick" in sys.argv
    os.makedirs(BUILD, exist_ok=True)
    orc = build_oracle()
    kvq = build_library()
    instrumented(orc)
    instrumented(kvq)
    oracle_tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    sel = ["not every and not all_fp32 and not sweep and not exhaust"] if quick else []
    rc1 = run_pytest(oracle_tests, {"KVQ_TEST_ORACLE_LIB": orc}, runtime("gcc"), sel)
    rc2 = run_pytest([os.path.join(ROOT, "tests", "test_boundary.py")],
                     {"KVQ_TEST_LIBKVQ": kvq, "KVQ_TEST_ORACLE_LIB": orc + ".unused"},
                     runtime("clang"))
    print(f"oracle tests under gcc ASan+UBSan: rc {rc1}; boundary tests under clang "
          f"ASan+UBSan: rc {rc2}", flush=True)
    return 0 if rc1 == 0 and rc2 == 0 else 1


if __name__ == "__main__":
    sys.exit(main())
