"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the CPU-side code.

- The oracle (plain C) is rebuilt with gcc's sanitizers and the whole pin
  suite (tests/test_oracle_pins.py) runs against that build.
- The library's host code (argument checks, policy, rotation tables,
  workspace layout, pyramid schedule, kept indices, byte accounting) is
  rebuilt with the sanitizers on the host side only -- device code is
  compiled as usual and never run -- and tests/abi_host_checks.c drives every
  reject path and host helper of include/kve.h through it, with no GPU.

Both fail on the first sanitizer report.  No GPU is used.
"""
from __future__ import annotations

import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "kv_cache_eviction_step_amd", "csrc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"gcc has no {name}")
    return path


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libkve_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c11", "-fPIC", "-shared",
                    "-ffp-contract=off", "-fno-fast-math", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-o", lib,
                    os.path.join(ROOT, "oracle", "kve_oracle.c"), "-lm"], check=True)
    env = dict(os.environ, **SAN_ENV, KVE_ORACLE_LIB=lib,
               LD_PRELOAD=_gcc_runtime("libasan.so") + ":" + _gcc_runtime("libubsan.so"))
    r = subprocess.run(["python", "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out


def _hip_tools():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    clang = "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not found")
    return hipcc, clang


def test_abi_host_side_under_asan_ubsan(tmp_path):
    hipcc, clang = _hip_tools()
    lib = str(tmp_path / "libkve_san.so")
    # sanitizers on the host side only: each -fsanitize= follows -Xarch_host
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=undefined",
                    "-Wno-unused-command-line-argument",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", lib,
                    os.path.join(CSRC, "kve_api.hip"), os.path.join(CSRC, "kve_step.hip")],
                   check=True, capture_output=True)
    exe = str(tmp_path / "abi_host_checks")
    # the driver is host-only C, linked with clang's sanitizer runtimes
    subprocess.run([clang, "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "abi_host_checks.c"),
                    "-o", exe, lib, f"-Wl,-rpath,{tmp_path}", "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib"], check=True)
    env = dict(os.environ, **SAN_ENV)
    env.pop("LD_PRELOAD", None)
    env["HIP_VISIBLE_DEVICES"] = "-1"          # never touch a GPU, even where one exists
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert out.startswith("ok: ") and "runtime error" not in out, out[-4000:]
