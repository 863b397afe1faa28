"""Build the HIP library (libgdr.so) in-tree for gfx950 with hipcc.

Every source is compiled to its own object (in parallel), then linked into
``linear_attention_chunked_amd/libgdr.so``.  ``build()`` always recompiles.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libgdr.so")
BUILD = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed-FP32 VALU forms are kept out of generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in arch VGPRs: the scan's state is also touched by VALU
    # every chunk, and the AGPR form would copy it back and forth
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]
SOURCES = ["scan.hip", "scan2.hip", "prepare.hip", "prepare2.hip", "output.hip", "output2.hip", "compose.hip", "abc.hip", "abc_out.hip", "kda.hip", "scan_bwd.hip", "plan.cpp", "api.cpp", "abc_api.cpp", "noalloc.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    lang = [] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [HIPCC, *COMMON, *lang, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = jobs or min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}", file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build()
