"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
C-ABI library's host side (plan creation, argument checks, every entry point
the CPU tests reach; the GPU code is built as usual) and the oracle are
rebuilt with -fsanitize=address,undefined, and the CPU suites that drive them
(ABI checks, binding checks, oracle pins) run against those builds in a child
process, any sanitizer report failing it.

Takes a few minutes (it compiles the library once more), so it runs only when
FCONV_SANITIZE=1:  FCONV_SANITIZE=1 python -m pytest tests/test_sanitizers.py"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "convolution_implicit_gemm_nhwc_amd", "csrc")
LLVM = "/opt/rocm/llvm"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(os.environ.get("FCONV_SANITIZE") != "1",
                                reason="set FCONV_SANITIZE=1 to build and run the sanitized host code")

SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]


def _host_only(flags):
    """Each sanitizer flag applies to the host compilation only."""
    out = []
    for f in flags:
        out += ["-Xarch_host", f]
    return out


def test_cpu_suites_under_asan_and_ubsan(tmp_path):
    runtime = glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux",
                                     "libclang_rt.asan-x86_64.so"))
    assert runtime, "clang's ASan runtime not found"
    objs = []
    for src in ("plan.cpp", "conv.hip", "wgrad.hip"):
        obj = str(tmp_path / (src + ".o"))
        cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
               "-fvisibility=hidden", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
        if src.endswith(".hip"):
            cmd += ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops"]
        cmd += _host_only(SAN) + ["-c", os.path.join(CSRC, src), "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True)
        objs.append(obj)
    lib = str(tmp_path / "libfconv_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *_host_only(SAN), *objs,
                    "-o", lib], check=True, capture_output=True)
    olib = str(tmp_path / "liboracle_san.so")
    subprocess.run([os.path.join(LLVM, "bin", "clang"), "-O1", "-g", "-fopenmp", "-ffp-contract=off",
                    "-fno-fast-math", "-std=c11", "-shared", "-fPIC", *SAN,
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", olib, "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=runtime[0], FCONV_LIBRARY=lib, FCONV_ORACLE_LIBRARY=olib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               LD_LIBRARY_PATH=os.path.join(LLVM, "lib") + ":" + os.environ.get("LD_LIBRARY_PATH", ""))
    env.pop("FCONV_SANITIZE", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", "tests/test_plan_abi.py", "tests/test_wgrad_abi.py",
                        "tests/test_binding_checks.py", "tests/test_oracle.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1800)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, report
