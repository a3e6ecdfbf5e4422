"""Build the HIP libraries in-tree with hipcc for gfx950.

Usage: ``python -m mla_decode_attention_split_amd.build`` (or call
:func:`build`).  Every HIP source is compiled with packed-fp32 instructions
disabled.  Two shared libraries are linked next to this file:

* ``libmla_decode.so`` -- the decode path (C ABI in include/mla_decode.h);
* ``libmla_ceiling.so`` -- the measurement probes the benchmark quotes the
  decode kernel against (C ABI in include/mla_ceiling.h); not linked by the
  decode library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_decode.so")
CEILING_LIB = os.path.join(HERE, "libmla_ceiling.so")
SOURCES = ["api.hip", "sched.hip", "decode.hip", "decode_wide.hip", "combine.hip"]
CEILING_SOURCES = ["ceiling.hip"]
ARCH = os.environ.get("MLA_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Per-source device-compiler options.  The main kernel keeps its MFMA
# accumulators in ordinary VGPRs (the rare rescale of O is then a plain
# multiply), which leaves the AGPRs free for operands the MFMAs read directly.
EXTRA = {
    "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "decode_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature; drop that notice
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


def _link(objs, lib):
    tmp = lib + ".tmp"
    _run(["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cmds = []

    def obj_of(s):
        return os.path.join(objdir, s.replace(".hip", ".o"))

    for s in SOURCES + CEILING_SOURCES:
        cmds.append(["hipcc", *COMMON, *EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", obj_of(s)])
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        list(ex.map(_run, cmds))
    _link([obj_of(s) for s in SOURCES], LIB)
    _link([obj_of(s) for s in CEILING_SOURCES], CEILING_LIB)
    if verbose:
        print("built", LIB, "and", CEILING_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
