"""Build libkvq.so (the HIP kernels and C ABI) in-tree for gfx950 with hipcc.

    python -m rotated_int2_kv_kvq_amd.build
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["abi.hip", "append.hip", "decode.hip"]
LIB = os.path.join(PKG, "libkvq.so")
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-fvisibility=hidden",
        "-Wl,--no-undefined",
        "-Wall",
        "-Wno-unused-command-line-argument",
        # a multiply feeds an add through one fma only where one expression
        # says so: a device function then rounds the same in every kernel that
        # inlines it (left to the back end, the fusion depends on the basic
        # blocks around it, and the staged and whole decode calls, or the
        # append and the fused decode step, would differ in the last bit)
        "-ffp-contract=on",
        # no packed fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{os.path.join(ROOT, 'include')}",
    ]


def scratch_users(remarks: str) -> list[str]:
    """Kernels whose resource-usage remarks report a private segment (register
    spills or stack) in the compiler's -Rpass-analysis=kernel-resource-usage
    output."""
    bad, name = [], None
    for ln in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", ln)
        if m and name and int(m.group(1)) > 0:
            bad.append(f"{name}: {m.group(1)} bytes/lane")
    return bad


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libkvq.so (always recompiles).  Fails when
    any kernel needs a private segment: a spill in the scan's loop would wait
    for every DMA in flight."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *flags(), "-Rpass-analysis=kernel-resource-usage",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    bad = scratch_users(res.stdout + res.stderr)
    if bad:
        raise RuntimeError("kernels with a private segment (register spills): " + "; ".join(bad))
    noise = [ln for ln in (res.stdout + res.stderr).splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "remark" not in ln
             and "kernel-resource-usage" not in ln
             and not re.match(r"\s*(\d+\s*)?\|", ln)]  # a remark's source excerpt
    if noise and verbose:
        print("\n".join(noise))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
