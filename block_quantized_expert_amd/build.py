"""Build libmoe.so in-tree: the HIP kernels for gfx950 plus the host-side
C ABI, with hipcc.  ``python -m block_quantized_expert_amd.build``."""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "lib", "libmoe.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_SOURCES = ["moe_api.hip", "moe_route_group.hip", "moe_ffn.hip", "moe_gemm.hip", "moe_fused.hip",
               "moe_pack.hip", "moe_probe.hip"]
HOST_SOURCES = ["moe_host.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I" + INCLUDE, "-I" + CSRC]
# Packed fp32 instructions are kept out of the device code on purpose.
HIP_FLAGS = COMMON + ["--offload-arch=" + ARCH, "-Xclang", "-target-feature",
                      "-Xclang", "-packed-fp32-ops"]
HOST_FLAGS = COMMON + ["-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # the host pass does not know the device-only feature above
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), "\n".join(lines)))
    return "\n".join(lines)


def build(verbose: bool = False) -> str:
    """Compile every source and link libmoe.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append((obj, [HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]))
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append((obj, ["g++"] + HOST_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]))
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        logs = list(ex.map(lambda j: _run(j[1]), jobs))
    tmp = LIB + ".tmp"
    logs.append(_run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH]
                     + [o for o, _ in jobs] + ["-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        for log in logs:
            if log:
                print(log)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
