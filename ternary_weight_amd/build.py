"""Build libbitlinear.so in-tree with hipcc for gfx950 only.

    python -m ternary_weight_amd.build

HIP sources are compiled with packed-fp32 instructions disabled
(-target-feature -packed-fp32-ops); host-only C++ is compiled by the same
driver without device code.  Objects go to ``_build/`` next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbitlinear.so")
ARCH = "gfx950"

HIP_SOURCES = ["quant.hip", "gemv.hip", "gemm.hip", "pack_device.hip", "api.hip", "probe.hip"]
CXX_SOURCES = ["pack.cpp", "gguf.cpp"]

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-result"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-ffp-contract=fast"]
CXX_FLAGS = ["-ffp-contract=off", "-pthread"]
# Per-source extras.  The decode kernel keeps its MFMA accumulators in
# ordinary VGPRs: its epilogue reads them with plain VALU operations instead
# of v_accvgpr_read copies.
EXTRA_FLAGS = {"gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _compile(cmd: list[str]) -> None:
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compile failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([hipcc, "-c", *COMMON, *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), os.path.join(CSRC, src),
                     "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([hipcc, "-c", *COMMON, *CXX_FLAGS, os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        for cmd, _ in zip(jobs, ex.map(_compile, jobs)):
            if verbose:
                print(" ".join(cmd))
    tmp = LIB + ".tmp"
    link = [hipcc, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-pthread", *objs, "-o", tmp]
    _compile(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
