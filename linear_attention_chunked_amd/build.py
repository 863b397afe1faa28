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


def resource_table(out_path: str, jobs: int | None = None) -> str:
    """Per-kernel resource use as the compiler reports it for gfx950
    (-Rpass-analysis=kernel-resource-usage on every source, the same flags as
    build()): VGPRs, AGPRs, SGPRs, scratch (spills), LDS and the occupancy in
    waves per SIMD those allow.  Writes a text table to ``out_path``."""
    import re
    import tempfile

    rows = []

    def one(src):
        path = os.path.join(CSRC, src)
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        with tempfile.TemporaryDirectory() as td:
            cmd = [HIPCC, *COMMON, *lang, "-Rpass-analysis=kernel-resource-usage", "-c", path, "-o",
                   os.path.join(td, "x.o")]
            r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(r.stderr[-2000:])
        cur, found = None, []
        for line in r.stderr.splitlines():
            m = re.search(r"remark:\s+(.*?):\s+(.*?) \[-Rpass-analysis", line)
            if not m:
                continue
            key, val = m.group(1).strip(), m.group(2).strip()
            if key == "Function Name":
                cur = {"kernel": val, "source": src}
                found.append(cur)
            elif cur is not None:
                cur[key] = val
        return found

    srcs = [s for s in SOURCES if s.endswith(".hip")]
    with cf.ThreadPoolExecutor(max_workers=jobs or min(8, os.cpu_count() or 4)) as ex:
        for found in ex.map(one, srcs):
            rows.extend(found)

    def demangle(names):
        r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
        return r.stdout.splitlines() if r.returncode == 0 else names

    names = demangle([r["kernel"] for r in rows])
    cols = [("VGPRs", "vgpr"), ("AGPRs", "agpr"), ("TotalSGPRs", "sgpr"), ("ScratchSize [bytes/lane]", "scratch"),
            ("VGPRs Spill", "vspill"), ("SGPRs Spill", "sspill"), ("LDS Size [bytes/block]", "lds_bytes"),
            ("Occupancy [waves/SIMD]", "waves/SIMD")]
    spilled = [n for r, n in zip(rows, names) if str(r.get("ScratchSize [bytes/lane]", "0")) != "0"]
    note = ("0 everywhere" if not spilled else
            f"0 except in {len(spilled)} kernel(s): " + "; ".join(n.split("(")[0].replace("void ", "") for n in spilled))
    lines = ["# Per-kernel resource use on gfx950 as the compiler reports it (-Rpass-analysis=kernel-resource-usage,",
             "# the library's own build flags); scratch = private memory per lane (register spills),",
             "# " + note,
             "#",
             "# command (from the repository root):",
             f"#   python -c 'from linear_attention_chunked_amd.build import resource_table; "
             f"resource_table(\"{os.path.relpath(out_path, ROOT)}\")'",
             "#",
             "# " + " ".join(f"{c[1]:>10}" for c in cols) + "  kernel (source)"]
    for r, name in sorted(zip(rows, names), key=lambda x: (x[0]["source"], x[1])):
        lines.append("  " + " ".join(f"{r.get(c[0], '?'):>10}" for c in cols) + f"  {name} ({r['source']})")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return out_path


if __name__ == "__main__":
    build()
