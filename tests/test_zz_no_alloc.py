"""gqa_attn_decode_noalloc on the GPU: the allocation-free decode (partials
in the library's fixed per-device scratch) against gqa_attn_decode with a
caller workspace -- the same kernels and split, so bit-identical -- and
against the fp64 oracle, on consecutive calls of different sizes (the
second smaller, so stale scratch from the first would show)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_ATOL_BF16, LSE_ATOL_F32, banner, check_bf16, check_f32, check_lse, np32
from gqa_flashattention_amd import binding as gq
from gqa_flashattention_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # (name, workload)
    ("decode_llama70b_32k", inputs.WORKLOADS["decode_llama70b_32k"]),
    ("ragged_b2", inputs.Workload("t", "decode", B=2, H_q=64, H_kv=8, d=128, dtype="bf16",
                                  lens=(5000, 3333), kv_cap=5120)),
    ("small_b1", inputs.Workload("t", "decode", B=1, H_q=64, H_kv=8, d=128, dtype="bf16",
                                 lens=(700,), kv_cap=768)),
    ("decode_small_f32", inputs.WORKLOADS["decode_small_f32"]),
]


def _both(x, w):
    out = torch.empty_like(x["q"])
    lse = torch.empty((w.B, w.H_q), dtype=torch.float32, device=DEV)
    gq.decode_noalloc(x["q"], x["k"], x["v"], x["kv_lens"], out, max_kv_len=max(w.lens),
                      scale=w.scale, lse=lse)
    ref_o, ref_l = gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], max_kv_len=max(w.lens),
                             scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    return out, lse, ref_o, ref_l


def test_decode_noalloc_matches_decode_on_consecutive_calls():
    """Each case in turn (sizes shrink after the first): bitwise equal to
    gqa_attn_decode, and within tolerance of the oracle."""
    for i, (name, w) in enumerate(CASES):
        banner("decode_noalloc", name, w.lens)
        x = inputs.make_decode(w, device=DEV, seed=900 + i)
        o, lse, ro, rl = _both(x, w)
        assert torch.equal(o, ro), f"{name}: O differs from gqa_attn_decode"
        assert torch.equal(lse, rl), f"{name}: LSE differs from gqa_attn_decode"
        want, want_l = oracle.decode(np32(x["q"]), np32(x["k"]), np32(x["v"]), np.array(w.lens),
                                     w.scale)
        if w.dtype == "f32":
            check_f32(np32(o), want, name)
            check_lse(np32(lse), want_l, name, LSE_ATOL_F32)
        else:
            for b in range(w.B):
                check_bf16(np32(o[b]), want[b], f"{name} seq {b}")
            check_lse(np32(lse), want_l, name, LSE_ATOL_BF16)


def test_decode_noalloc_rejects_oversized_call():
    """A call whose partials exceed the fixed scratch is refused before any
    launch, and the output is left untouched."""
    w = inputs.Workload("t", "decode", B=8, H_q=64, H_kv=8, d=128, dtype="bf16",
                        lens=(1024,) * 8, kv_cap=1024)
    banner("decode_noalloc_oversized")
    x = inputs.make_decode(w, device=DEV, seed=910)
    out = torch.full_like(x["q"], 7.0)
    with pytest.raises(gq.GQAError) as e:
        gq.decode_noalloc(x["q"], x["k"], x["v"], x["kv_lens"], out, max_kv_len=131072 * 2,
                          scale=w.scale)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
