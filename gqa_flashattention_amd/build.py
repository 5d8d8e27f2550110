"""Build the gfx950 HIP library ``libgqa_attn.so`` in-tree with hipcc.

Usage: ``python -m gqa_flashattention_amd.build`` (or ``build()`` from
Python).  Each ``csrc/*.hip`` file is compiled to an object in parallel, then
linked into a shared library next to this file.  All device code is built
for gfx950 only, with packed-fp32 instruction generation disabled.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgqa_attn.so")
SOURCES = ["api.hip", "decode.hip", "decode_multi.hip", "merge.hip", "prefill.hip"]

DEVICE_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


# Per-source flags.  decode.hip, decode_multi.hip: kernel-argument
# preloading (gfx950 loads the first kernel arguments into registers at wave
# launch; these files' kernels put the values their first loads need first,
# so those loads do not wait for the argument block).  Where the firmware
# does not preload, a kernel starts with a fallback that loads those
# arguments itself.
SOURCE_FLAGS = {
    "decode.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=5"],
    "decode_multi.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=4"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-I", INCLUDE, "-I", CSRC, "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    """Compile every HIP source and link ``libgqa_attn.so``; return its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
