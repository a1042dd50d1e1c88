"""Build libzero_partition.so (HIP kernels + C ABI) and libzero_probe.so (the
achievable-bandwidth probes the benchmark reports beside the step) for gfx950
with hipcc.

Run `python -m sharded_zero_partition_amd.build` (or call build()).  Objects
go to _build/ at the repository root; the shared libraries are written next
to this file, where the Python bindings load them.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libzero_partition.so")
PROBE_LIB = os.path.join(PKG, "libzero_probe.so")

SOURCES = ["layout.cpp", "capi.cpp", "pack.hip", "shard_step.hip", "reduce_owner.hip", "noalloc.hip"]
PROBE_SOURCES = ["stream_probe.hip"]

ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
    # one rounding per written fp32 operation: no fused multiply-add
    # contraction, IEEE division and square root (hipcc's default), no fast-math
    "-ffp-contract=off", "-fno-fast-math",
]

# packed fp32 instructions stay off: the compiler may only emit scalar fp32 ALU ops
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          ]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    subprocess.run(cmd, check=True)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
