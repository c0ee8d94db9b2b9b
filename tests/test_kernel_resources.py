"""Every kernel of the library compiles for gfx950 without vector-register
spills or scratch memory.

A vector-register spill puts per-lane scratch traffic into a loop that the
design keeps in registers. It can appear silently when a shared body gains an
instantiation (an fp8 variant, an unrolled loop), so every HIP source is
compiled device-only with the compiler's resource-usage remarks, using the
library's own flags. The test then checks each kernel's VGPR spill count and
scratch size. Scalar-register spills go to lanes of a vector register, touch
no memory, and sit in kernel set-up code, so they are allowed. Compilation
only: no GPU is needed.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from dynamic_column_sparse_amd import build

REMARK = re.compile(r"remark:\s+(Function Name|VGPRs Spill|ScratchSize \[bytes/lane\]):\s+(\S+)")


def _resources(src):
    cmd = [build.hipcc(), "-x", "hip", "--cuda-device-only", *build.common_flags(), "-w",
           "-DCHIPMUNK_SOURCE_DIGEST=\"test\"", "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(build.CSRC, src), "-o", os.devnull]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{src}: hipcc failed\n{r.stderr[-3000:]}"
    kernels, cur = {}, None
    for key, val in REMARK.findall(r.stderr):
        if key == "Function Name":
            cur = kernels.setdefault(val, {})
        elif cur is not None:
            cur[key] = val
    return src, kernels


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_no_kernel_spills_vector_registers_or_uses_scratch():
    srcs = [s for s in build.SOURCES if s.endswith(".hip")]
    with ThreadPoolExecutor(min(len(srcs), 8)) as ex:
        results = list(ex.map(_resources, srcs))
    total, bad = 0, []
    for src, kernels in results:
        for name, res in kernels.items():
            total += 1
            vspill, scratch = int(res.get("VGPRs Spill", 0)), int(res.get("ScratchSize [bytes/lane]", 0))
            if vspill or scratch:
                bad.append(f"{src}: {name} VGPR spill {vspill}, scratch {scratch} B/lane")
    assert total >= 30, f"expected the library's kernels, found {total}"
    assert not bad, "\n".join(bad)
