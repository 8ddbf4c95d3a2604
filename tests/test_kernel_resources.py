"""Compile-time resource check of the HIP kernels (CPU only, needs hipcc).

Every kernel is compiled for gfx950 with the library's own flags and the
compiler's resource report; a kernel that uses scratch memory (stack or
register spills) fails here unless listed below. Scratch in a hot loop costs
several times the kernel's run time, and it can appear silently when a
lambda holding register arrays by reference stays out of line.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from varlen_gqa_attention_amd import build as B

# Kernels allowed to use scratch memory (none at present).
ALLOWED = re.compile(r"^$")

KERNEL_SOURCES = ["decode.hip", "prefill.hip", "mask.hip", "bwd.hip", "noalloc.hip"]


def _report(src):
    hipcc = B._hipcc()
    cmd = [hipcc, *B._flags(), "-x", "hip", "--cuda-device-only", "-c",
           os.path.join(B.CSRC, src), "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    usage, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]): (\S+)", line)
        if not m:
            continue
        if m.group(1) == "Function Name":
            name = m.group(2)
        else:
            usage[name] = int(m.group(2))
    return usage


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_no_kernel_uses_scratch_memory():
    with cf.ThreadPoolExecutor(max_workers=len(KERNEL_SOURCES)) as ex:
        reports = list(ex.map(_report, KERNEL_SOURCES))
    usage = {k: v for r in reports for k, v in r.items()}
    assert any("prefill_kernel" in k for k in usage) and any("bwd_dkdv" in k for k in usage)
    bad = {k: v for k, v in usage.items() if v > 0 and not ALLOWED.search(k)}
    assert not bad, f"kernels using scratch memory: {bad}"
