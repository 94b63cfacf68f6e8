"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the C ABI layer (argument validation, workspace arithmetic) and the C
oracle are rebuilt with clang's sanitizers, and the boundary and oracle-pin
tests run against those builds in a child process with the sanitizer runtime
preloaded.  Any report fails the test.  The HIP kernel objects are linked
unchanged (no device code is sanitized, and no GPU is used)."""
import glob
import os
import subprocess
import sys

import pytest

from conftest import ROOT

LLVM = "/opt/rocm/llvm/bin"
PKG = os.path.join(ROOT, "softmax_free_score_amd")
OBJ = os.path.join(PKG, "_build")
OUT = os.path.join(OBJ, "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def _build():
    os.makedirs(OUT, exist_ok=True)
    kernels = sorted(o for o in glob.glob(os.path.join(OBJ, "*.o"))
                     if os.path.basename(o) != "attn_api.o")
    if not kernels:
        pytest.skip("the HIP objects are not built (python -m softmax_free_score_amd.build)")
    api_o = os.path.join(OUT, "attn_api.o")
    # host-only C++: the HIP runtime API is declared by its headers
    _run([f"{LLVM}/clang++", "-x", "c++", "-std=c++17", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__",
          "-I/opt/rocm/include", f"-I{ROOT}/include", f"-I{PKG}/csrc",
          "-c", os.path.join(PKG, "csrc", "attn_api.cpp"), "-o", api_o])
    lib = os.path.join(OUT, "libsfs_attn.so")
    _run([f"{LLVM}/clang++", "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan",
          api_o, *kernels, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
          "-o", lib])
    oracle_lib = os.path.join(OUT, "liboracle.so")
    _run([f"{LLVM}/clang", "-std=c11", "-fPIC", "-shared", "-fopenmp", *SAN,
          os.path.join(ROOT, "oracle", "attn_oracle.c"), "-o", oracle_lib, "-lm",
          f"-L{os.path.dirname(LLVM)}/lib", f"-Wl,-rpath,{os.path.dirname(LLVM)}/lib"])
    runtime = _run([f"{LLVM}/clang", "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()
    if not os.path.exists(runtime):
        runtime = glob.glob(f"{os.path.dirname(LLVM)}/lib/clang/*/lib/*/libclang_rt.asan*x86_64*.so")
        runtime = runtime[0] if runtime else ""
    assert os.path.exists(runtime), "clang's ASan runtime is missing"
    return lib, oracle_lib, runtime


def test_boundary_and_oracle_pins_under_sanitizers():
    if not os.path.exists(f"{LLVM}/clang++"):
        pytest.skip("ROCm's clang is not installed")
    lib, oracle_lib, runtime = _build()
    env = dict(os.environ)
    env.update(SFS_ATTN_LIBRARY=lib, SFS_ORACLE_LIBRARY=oracle_lib, LD_PRELOAD=runtime,
               # the interpreter itself is not instrumented and keeps memory to the end
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", "tests/test_boundary.py",
                        "tests/test_oracle_pins.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error:" not in text, text[-6000:]
    assert r.returncode == 0, text[-6000:]
    assert " passed" in r.stdout
