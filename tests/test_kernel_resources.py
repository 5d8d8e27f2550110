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
    cmd = [build.hipcc(), *build.DEVICE_FLAGS, *build.SOURCE_FLAGS.get(src, []), "-I", build.INCLUDE,
           "-I", build.CSRC, "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o",
           str(tmp_path / "out.s"), "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", r.stderr)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
    assert names and len(names) == len(scratch), "resource report not found"
    bad = [(n, sc) for n, sc in zip(names, scratch) if sc > ALLOWED_SCRATCH.get(n, 0)]
    assert not bad, f"kernels using scratch memory: {bad}"


@pytest.mark.parametrize("src", [s for s in build.SOURCES if s != "api.hip"])
def test_m0_only_in_lds_dma_sequences(src, tmp_path):
    """M0 holds the LDS destination of the direct global -> LDS loads, which
    are issued as inline assembly.  The compiler reserves M0 (it cannot be
    declared clobbered), so check the generated code instead: every
    instruction that names M0 is one of those sequences' `s_mov_b32 m0`,
    followed (after at most one s_nop) by its `buffer_load ... lds`.  Any
    other use would mean the compiler keeps a value of its own in M0 that
    the sequence could overwrite."""
    out = tmp_path / "out.s"
    cmd = [build.hipcc(), *build.DEVICE_FLAGS, *build.SOURCE_FLAGS.get(src, []), "-I", build.INCLUDE,
           "-I", build.CSRC, "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln.split(";")[0].strip() for ln in out.read_text().splitlines()]
    lines = [ln for ln in lines if ln and not ln.startswith((".", "//"))]
    bad = []
    for i, ln in enumerate(lines):
        if not re.search(r"\bm0\b", ln):
            continue
        nxt = [x for x in lines[i + 1:i + 3] if x != "s_nop 0"]
        ok = (re.fullmatch(r"s_mov_b32 m0, s\d+", ln) is not None and nxt
              and re.match(r"buffer_load_dword\S* .* lds$", nxt[0]) is not None)
        if not ok:
            bad.append((i, ln))
    assert not bad, f"M0 used outside the LDS DMA sequences: {bad[:5]}"


def test_decode_leading_arguments_preloaded(tmp_path):
    """The decode split kernels (bf16 and fp32) and the combine kernel take
    the values their first loads need as leading kernel arguments; the build
    preloads them into registers (and keeps the other arguments in memory)."""
    out = tmp_path / "out.s"
    cmd = [build.hipcc(), *build.DEVICE_FLAGS, *build.SOURCE_FLAGS.get("decode.hip", []), "-I",
           build.INCLUDE, "-I", build.CSRC, "--cuda-device-only", "-S",
           os.path.join(build.CSRC, "decode.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = out.read_text()
    found = dict(re.findall(r"\.amdhsa_kernel (\S+)\n(?:.*\n)*?\s*\.amdhsa_user_sgpr_kernarg_preload_length (\d+)",
                            text))
    split = [n for n in found if "decode_partial_bf16_kernel" in n or "decode_partial_f32_kernel" in n]
    comb = [n for n in found if "decode_combine_kernel" in n]
    assert len(split) == 6 and len(comb) == 6, found
    assert all(int(found[n]) == 2 for n in split), found        # the length pointer
    assert all(int(found[n]) == 8 for n in comb), found         # 3 pointers, 2 ints


def test_multi_token_leading_arguments_preloaded(tmp_path):
    """The multi-token split kernel's leading arguments (the length pointer,
    Q, H_kv and the fold's rows) are preloaded into registers."""
    out = tmp_path / "out.s"
    cmd = [build.hipcc(), *build.DEVICE_FLAGS, *build.SOURCE_FLAGS.get("decode_multi.hip", []), "-I",
           build.INCLUDE, "-I", build.CSRC, "--cuda-device-only", "-S",
           os.path.join(build.CSRC, "decode_multi.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    found = dict(re.findall(r"\.amdhsa_kernel (\S+)\n(?:.*\n)*?\s*\.amdhsa_user_sgpr_kernarg_preload_length (\d+)",
                            out.read_text()))
    multi = [n for n in found if "decode_multi_partial_kernel" in n]
    assert len(multi) == 6 and all(int(found[n]) == 6 for n in multi), found
