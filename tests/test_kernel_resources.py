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


# Known, harmless scratch: the prefill kernel (dense, varlen and paged forms) keeps
# a few dwords (the 64-bit output row index that addresses O and the LSE,
# and other epilogue values) live across its main loop without using them
# inside it; they are stored once before the loop and reloaded once after
# it (the listing is checked by hand when this changes).
ALLOWED_SCRATCH = {f"_ZN3gqa19prefill_bf16_kernelILb{v}ELb{pg}EEEvNS_13PrefillParamsE": 40
                   for v, pg in ((0, 0), (1, 0), (1, 1))}


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
