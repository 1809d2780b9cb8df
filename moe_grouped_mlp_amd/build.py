"""Build libmoe_gmlp.so (gfx950) in-tree with hipcc.

    python -m moe_grouped_mlp_amd.build      # or __graft_entry__.build()

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection switched off, then linked into one shared library next to this
file.  Objects go to moe_grouped_mlp_amd/_build/.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_gmlp.so")

SOURCES = ["api.cpp", "route.hip", "router.hip", "unfused.hip", "permute.hip", "quant.hip", "gemm.hip", "gemm_store.hip",
           "gemm_glu_bf16.hip", "gemm_glu_mx.hip", "gemm_dglu_bf16.hip", "gemm_dglu_mx.hip", "gemm_wgrad.hip",
           "gemm_store_mx4.hip", "gemm_glu_mx4.hip", "gemm_dglu_mx4.hip", "gemm_wgrad_mx4.hip",
           "noalloc.hip",
           "router_route.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Wall", "-Wno-unused-function",
    # never select packed fp32 VALU instructions (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature: drop that note
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found ({HIPCC})")
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
