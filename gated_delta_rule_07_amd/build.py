"""Build libkda.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m gated_delta_rule_07_amd.build`` (or ``build()`` from Python).
Each source compiles to an object in parallel, then one shared library is linked
next to this file.  hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
INCLUDE = PKG.parent / "include"
LIB = PKG / "libkda.so"
TEST_LIB = PKG / "libkda_testhooks.so"
OBJDIR = PKG / "_build"

SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_prefill.hip", "kda_prefill_pipe.hip", "kda_prep.hip",
           "kda_spec.hip", "kda_split.hip"]

ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled: plain fp32 code only.  Matrix-core
# accumulators stay in ordinary VGPRs: with one wave per SIMD the compiler would
# otherwise park them in AccVGPRs and copy them out for every VALU use.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; libkda needs ROCm to build")
    return path


def _compile(src: str, verbose: bool, defines=()) -> Path:
    out = OBJDIR / (Path(src).stem + ("_hooks" if defines else "") + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *defines, "-c", str(CSRC / src), "-o", str(out)]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return out


def _link(objs, lib: Path, verbose: bool) -> None:
    tmp = lib.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *map(str, objs), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int | None = None) -> Path:
    """Compile every source and link libkda.so; always rebuilds.

    Also links libkda_testhooks.so: the same kernels with the C ABI compiled
    with KDA_TEST_HOOKS, which adds kda_test_force_prefill (the tests use it to
    run the generic kernel on shapes the pipelined kernel would serve).  The
    product library carries no such switch."""
    OBJDIR.mkdir(exist_ok=True)
    jobs = jobs or min(len(SOURCES) + 1, max(1, os.cpu_count() or 1))
    units = [(s, ()) for s in SOURCES] + [("kda_api.cpp", ("-DKDA_TEST_HOOKS",))]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u[0], verbose, u[1]), units))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link([objs[-1]] + objs[1:len(SOURCES)], TEST_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
