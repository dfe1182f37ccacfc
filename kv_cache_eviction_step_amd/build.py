"""Build libkve.so (the C-ABI library) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkve.so")
SOURCES = ["kve_api.hip", "kve_step.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-ffp-contract=fast-honor-pragmas",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


# Every kernel must keep two 512-thread workgroups (or one 1024-thread
# workgroup) per compute unit (4 waves per SIMD, i.e. at most 128 VGPRs) and
# must not spill VGPRs to scratch memory.
MIN_WAVES_PER_SIMD = 4
# ... except the per-layer kernel for launches of at most one workgroup per
# compute unit, which needs room for one 512-thread workgroup (2 waves per SIMD)
SOLO_KERNEL = "step_kernel_solo"
MIN_WAVES_PER_SIMD_SOLO = 2


def kernel_resources(remarks: str) -> dict[str, dict[str, int]]:
    """Per-kernel figures from hipcc's -Rpass-analysis=kernel-resource-usage remarks."""
    out: dict[str, dict[str, int]] = {}
    cur = None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(VGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]"
                      r"|VGPRs Spill|SGPRs Spill): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).split(" [")[0]] = int(m.group(2))
    return out


def check_resources(res: dict[str, dict[str, int]]) -> list[str]:
    bad = []
    for name, r in res.items():
        if "kernel" not in name:
            continue
        # (an SGPR spill goes to a VGPR lane, not to memory: allowed)
        need = MIN_WAVES_PER_SIMD_SOLO if SOLO_KERNEL in name else MIN_WAVES_PER_SIMD
        if (r.get("Occupancy", 0) < need or r.get("ScratchSize", 0) or
                r.get("VGPRs Spill", 0)):
            bad.append(f"{name}: {r}")
    return bad


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str = LIB,
          check: bool = True) -> str:
    """Compile libkve.so.  With `check`, fail if a kernel spills or drops below
    MIN_WAVES_PER_SIMD (tuning builds with other launch shapes pass check=False)."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []),
           "-Rpass-analysis=kernel-resource-usage",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to build libkve.so")
    res = kernel_resources(r.stderr)
    if check:
        if not any("kernel" in k for k in res):
            raise RuntimeError("hipcc printed no kernel resource usage")
        bad = check_resources(res)
        if bad:
            raise RuntimeError("kernel resource check failed:\n  " + "\n  ".join(bad))
    if verbose:
        for name, fig in sorted(res.items()):
            if "kernel" in name:
                print(f"{name}: {fig}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
