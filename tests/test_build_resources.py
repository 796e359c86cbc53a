"""The hot-path kernels compile for gfx950 without register spills.

A spill (scratch memory per lane) in one of the GEMM, attention, tree or draft kernels
costs 5-15% of its time, and it can appear from an unrelated change: the epilogues are
inlined into every GEMM instance, so one more epilogue variant has pushed the widest tile
configurations over 256 VGPRs before.  hipcc's resource-usage remarks report the scratch
size of every kernel; this test compiles each source (CPU only, no GPU needed) and
requires zero scratch everywhere."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from tree_attention_verification_06_amd.build import ARCH, CSRC, HERE, HIPCC

SOURCES = ["gemm.hip", "attn.hip", "tree.hip", "draft.hip", "decode.hip"]


def _remarks(src):
    cmd = [HIPCC, "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I" + os.path.join(HERE, "..", "include"), "--cuda-device-only", "-c",
           os.path.join(CSRC, src), "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stderr


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_no_kernel_spills_registers():
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        outs = dict(zip(SOURCES, ex.map(_remarks, SOURCES)))
    bad = []
    n = 0
    for src, text in outs.items():
        name = None
        for line in text.splitlines():
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                name = m.group(1)
            m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
            if m:
                n += 1
                if int(m.group(1)) != 0:
                    bad.append((src, name, int(m.group(1))))
    assert n >= 20, "no resource-usage remarks found"
    assert not bad, f"kernels with scratch: {bad}"
