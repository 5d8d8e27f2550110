"""Every gfx950 kernel compiles without private (scratch) memory: no register
spills and no kernel state in stack memory (CPU only; hipcc cross-compiles).

A spill or a non-inlined helper silently moves kernel state to scratch and
costs a large part of the bandwidth, so this is checked on every source."""

import os
import re
import shutil
import subprocess

import pytest

from gqa_flashattention_amd import build

pytestmark = pytest.mark.skipif(shutil.which(build.hipcc()) is None and not os.path.exists(build.hipcc()),
                                reason="hipcc not available")


# No kernel may use scratch: the prefill kernel re-derives its output
# addressing after the main loop (from the workgroup id and the kernel
# arguments) instead of keeping it live through the loop.
ALLOWED_SCRATCH = {}


@pytest.mark.parametrize("src", build.SOURCES)
def test_no_scratch(src, tmp_path):
    if src == "api.hip":
        pytest.skip("host code only")
    cmd = [build.hipcc(), *build.DEVICE_FLAGS, "-I", build.INCLUDE, "-I", build.CSRC,
           "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o",
           str(tmp_path / "out.s"), "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", r.stderr)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
    assert names and len(names) == len(scratch), "resource report not found"
    bad = [(n, sc) for n, sc in zip(names, scratch) if sc > ALLOWED_SCRATCH.get(n, 0)]
    assert not bad, f"kernels using scratch memory: {bad}"
