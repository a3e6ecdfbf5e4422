"""Register budget of every decode-kernel instance: no scratch memory.

The decode kernels keep their whole state (query fragments, output
accumulators, softmax state, page lists) in registers and LDS; a spill to
scratch would put memory waits into the stage loop, where a vector-memory
wait also drains the prefetched stages.  This test compiles the kernel
sources for gfx950 (device code only, the flags the build uses) and reads the
compiler's per-kernel metadata.  It needs hipcc but no GPU.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from mla_decode_attention_split_amd import build

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not installed")

KERNEL_SOURCES = ["decode.hip", "decode_wide.hip"]


def _kernel_metadata(src, outdir):
    out = os.path.join(outdir, src.replace(".hip", ".s"))
    flags = [f for f in build.COMMON if f not in ("-fPIC", "-Wall", "-Wno-unused-function")]
    cmd = ["hipcc", *flags, *build.EXTRA.get(src, []), "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    text = open(out).read()
    # the AMDGPU metadata block lists each kernel's fields, then its .name
    kernels = {}
    for block in re.split(r"\n\s+- \.", text.split("amdhsa.kernels:")[1]):
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name or "decode_kernel" not in name.group(1):
            continue
        fields = {k: int(v) for k, v in re.findall(r"\.(private_segment_fixed_size|vgpr_spill_count|"
                                                    r"agpr_count|vgpr_count):\s+(\d+)", block)}
        kernels[name.group(1)] = fields
    return kernels


def test_decode_kernels_use_no_scratch(tmp_path):
    with ThreadPoolExecutor(max_workers=2) as ex:
        parts = list(ex.map(lambda s: _kernel_metadata(s, str(tmp_path)), KERNEL_SOURCES))
    kernels = {k: v for p in parts for k, v in p.items()}
    # 16/32/64-row tiles with one or several KV heads, the 128-row tile with
    # one; the 16- and 32-row tiles with both key-stage cache policies; each
    # in bf16 and fp16
    assert len(kernels) == 22, sorted(kernels)
    for name, f in kernels.items():
        assert f.get("private_segment_fixed_size") == 0, (name, f)
        assert f.get("vgpr_spill_count") == 0, (name, f)
