"""Builds libctr.so (HIP for gfx950) in-tree with hipcc.

    python -m sparse_embedding_lookup_amd.build

Every kernel must keep its values in registers: the build fails when the compiler's resource
report gives any kernel scratch memory (a register array it could not keep in registers, or
spills), which on these kernels has meant loads issued one at a time.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libctr.so")
OBJ = os.path.join(HERE, "_build")

SOURCES = ["capi.cpp", "step.cpp", "unique.hip", "embbag.hip", "segreduce.hip", "interaction.hip",
           "dict.hip", "dense.hip", "fused.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _scratch_kernels(report: str) -> list:
    """Kernels with a nonzero ScratchSize in hipcc's kernel-resource-usage remarks."""
    out, name = [], None
    for line in report.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            out.append("%s (%s bytes per lane)" % (name, m.group(1)))
    return out


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, src + ".o")
    report = ["-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + report + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    scratch = _scratch_kernels(r.stderr)
    if scratch:
        raise RuntimeError("kernels of %s use scratch memory:\n  %s" % (src, "\n  ".join(scratch)))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
