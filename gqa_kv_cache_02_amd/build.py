"""Build libgqa.so (HIP, gfx950) in-tree with hipcc.

    python -m gqa_kv_cache_02_amd.build

Every translation unit is compiled for gfx950 only, with packed-fp32 VALU
instructions disabled, then linked into gqa_kv_cache_02_amd/libgqa.so.

The compiler's resource report for each HIP file is checked: every device
function it lists must be a kernel (nothing compiled out of line into a
called function) and use no scratch memory.  A kernel whose tile math was
split into called functions reached its operands through pointers into
scratch; two such prefill variants faulted the GPU, so the build refuses
that form outright.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgqa.so")

SOURCES = ["gqa_api.cpp", "gqa_generic.hip", "gqa_decode.hip", "gqa_prefill.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


REMARK = "-Rpass-analysis=kernel-resource-usage"
_KERNEL = re.compile(r"^_ZN3gqa\d+[a-z0-9_]*_kernelI")


def resource_violations(report: str) -> list[str]:
    """Device functions in a compiler resource report that are not kernels,
    or that use scratch memory.  `report` is hipcc's stderr with REMARK on."""
    out = []
    name = None
    for ln in report.splitlines():
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
            if not _KERNEL.match(name):
                out.append(f"{name}: a called device function (tile math compiled out of line)")
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", ln)
        if m and name is not None and int(m.group(1)) > 0:
            out.append(f"{name}: {m.group(1)} bytes of scratch per lane")
    return out


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    hip = src.endswith(".hip")
    # (no source excerpts under the remarks: they would bury real warnings)
    extra = [REMARK, "-fno-caret-diagnostics"] if hip else []
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    if hip:
        bad = resource_violations(res.stderr)
        if bad:
            raise RuntimeError(f"{src}: every kernel must run without calls and without "
                               "scratch:\n  " + "\n  ".join(bad))
    # hipcc's host pass does not know the packed-fp32 target feature; that
    # warning is expected, anything else (but the resource report) is shown.
    noise = ("'-packed-fp32-ops' is not a recognized feature", REMARK)
    msgs = [ln for ln in res.stderr.splitlines()
            if ln.strip() and not any(n in ln for n in noise)]
    if msgs:
        print(f"[{src}]\n" + "\n".join(msgs), file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
