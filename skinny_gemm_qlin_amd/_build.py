"""Build libqlin.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Flags:
  --offload-arch=gfx950                 CDNA4 only, no other code objects
  -O3 -std=c++17 -fPIC
  -fhip-fp32-correctly-rounded-divide-sqrt
                                        IEEE division in the INT8 quantiser
  -fno-gpu-flush-denormals-to-zero      keep fp32 subnormals (UE8M0 byte 0)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                        no packed-fp32 VALU instructions
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqlin.so")

SOURCES = ["gemv.hip", "ks_i8.hip", "ks_f8.hip", "ks_w8a8_e4m3.hip", "ks_w8a8_e5m2.hip", "qlin_api.hip",
           "act_quant.hip", "gemm.hip", "moe.hip", "moe_prefill.hip", "routing.hip"]
HEADERS = ["qlin_device.hpp", "qlin_launch.hpp", "gemv_kernels.hpp", "mfma_kernels.hpp", "ks_kernels.hpp",
           "ks_launch.hpp", "gemm_kernels.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libqlin.so next to this file."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
