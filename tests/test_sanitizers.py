"""Sanitizer tier (CPU only): AddressSanitizer and UndefinedBehaviorSanitizer
builds of the oracle and of the libkda C ABI's host code, each driven by a small
program under tests/sanitize/ that must run clean.

* The oracle is built with gcc; its driver runs every entry point over every
  input dtype, head selection, column blocking and thread count, the worked
  example, and the argument rejections.
* The C ABI (argument validation, aliasing checks, kernel choice and the
  planning queries) is compiled with hipcc for the host only with the
  sanitizers, and linked with the kernel objects of the regular in-tree build;
  its driver makes only calls that validation refuses, plus host-only queries,
  so nothing is ever launched.

Sanitizer flags apply to host code only (each -fsanitize= follows -Xarch_host
on a hipcc line).
"""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SAN = ROOT / "tests" / "sanitize"
BUILD = ROOT / "gated_delta_rule_07_amd" / "_build"
KERNEL_OBJS = ["kda_decode.o", "kda_prefill.o", "kda_prefill_pipe.o", "kda_prep.o", "kda_spec.o", "kda_split.o"]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    exe = tmp_path / "oracle_san"
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-pthread", str(SAN / "oracle_main.c"), str(ROOT / "oracle" / "kda_oracle.c"),
          "-o", str(exe), "-lm"])
    r = _run([str(exe)], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert "clean" in r.stdout


def test_c_abi_validation_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    objs = [BUILD / o for o in KERNEL_OBJS]
    if not all(o.exists() for o in objs):
        pytest.skip("kernel objects not built (python -m gated_delta_rule_07_amd.build)")
    common = ["-x", "hip", "--offload-host-only", "-O1", "-g", "-std=c++17", f"-I{ROOT / 'include'}",
              f"-I{ROOT / 'gated_delta_rule_07_amd' / 'csrc'}", *HOST_SAN]
    api_o, main_o, exe = tmp_path / "api.o", tmp_path / "main.o", tmp_path / "api_san"
    # kda_api.cpp holds a device array (the allocation-free entry point's scratch):
    # its device part is built too, the sanitizers apply to the host part only
    api_flags = [f for f in common if f != "--offload-host-only"] + ["--offload-arch=gfx950"]
    _run([hipcc, *api_flags, "-c", str(ROOT / "gated_delta_rule_07_amd" / "csrc" / "kda_api.cpp"), "-o", str(api_o)])
    _run([hipcc, *common, "-c", str(SAN / "api_main.cpp"), "-o", str(main_o)])
    _run([hipcc, *HOST_SAN, "--offload-arch=gfx950", str(main_o), str(api_o), *map(str, objs), "-o", str(exe)])
    # the HIP runtime's own allocations at load are not ours to judge: leaks off
    r = _run([str(exe)], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    assert "clean" in r.stdout and "runtime error" not in r.stderr
