"""Build ``libsfs_attn.so`` in-tree with hipcc for gfx950.

    python -m softmax_free_score_amd.build

Compiles the C-ABI layer and the HIP kernels (the bf16 kernel once per key
width) in parallel and links one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsfs_attn.so")
ARCH = "gfx950"

# Packed fp32 instructions are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return exe


def _units():
    units = [("attn_api", "attn_api.cpp", [])]
    units.append(("attn_f32", "attn_f32.hip", []))
    units.append(("attn_combine", "attn_combine.hip", []))
    units.append(("attn_bwd_aux", "attn_bwd_aux.hip", []))
    units.append(("attn_scratch", "attn_scratch.hip", []))
    for dk in (16, 32, 64, 128):
        units.append((f"attn_bf16_dk{dk}", "attn_bf16.hip", [f"-DSFS_DK={dk}"]))
        units.append((f"attn_bwd_dk{dk}", "attn_bwd.hip", [f"-DSFS_DK={dk}"]))
        units.append((f"attn_decode_dk{dk}", "attn_decode.hip", [f"-DSFS_DK={dk}"]))
        units.append((f"attn_telemetry_dk{dk}", "attn_telemetry.hip", [f"-DSFS_DK={dk}"]))
    return units


def _compile(hipcc, name, src, defs, verbose):
    out = os.path.join(OBJ, name + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [hipcc, "-x", "hip", f"--offload-arch={ARCH}", *DEVICE_FLAGS, *COMMON, *defs,
               "-c", path, "-o", out]
    else:
        cmd = [hipcc, *COMMON, *defs, "-c", path, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} {' '.join(defs)} failed:\n{err}")
    if err.strip() and verbose:
        print(err)
    return out


def build(verbose: bool = False, jobs: int | None = None, extra_defs=(), out: str | None = None,
          obj_dir: str | None = None) -> str:
    """Compile and link; ``extra_defs`` are added to every kernel unit (e.g.
    ``-DSFS_NW=8`` to change the launch shape), ``out`` overrides the library
    path."""
    global OBJ
    hipcc = _hipcc()
    OBJ = obj_dir or OBJ
    os.makedirs(OBJ, exist_ok=True)
    units = [(n, s, d + list(extra_defs)) for n, s, d in _units()]
    jobs = jobs or min(len(units), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda u: _compile(hipcc, *u, verbose), units))
    lib = out or LIB
    tmp = lib + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
