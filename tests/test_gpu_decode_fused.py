"""gqa_attn_decode_fused on the GPU: the one-launch decode whose last
arriving split workgroup of each (sequence, KV head) merges the partials.
It runs the combine launch's merge code in the same order, so it must equal
gqa_attn_decode bit for bit for the same split, and the fp64 oracle within
the stated tolerances; its arrival counters must come back to zero after
every call, so repeated calls on one workspace stay bit-identical."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (LSE_ATOL_BF16, LSE_ATOL_F32, banner, check_bf16, check_f32, check_lse,
                      np32)
from gqa_flashattention_amd import binding as gq
from gqa_flashattention_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(x, w, chunk=0, ws=None, reps=1):
    kw = dict(max_kv_len=max(w.lens), scale=w.scale, chunk_tokens=chunk, return_lse=True)
    ref_o, ref_l = gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], **kw)
    outs = [gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], workspace=ws, phase="fused", **kw)
            for _ in range(reps)]
    torch.cuda.synchronize()
    return ref_o, ref_l, outs


def _check_oracle(o, lse, x, w, what):
    ro, rl = oracle.decode(np32(x["q"]), np32(x["k"]), np32(x["v"]), x["kv_lens"].cpu().numpy(),
                           w.scale)
    if w.dtype == "f32":
        check_f32(np32(o), ro, what)
        check_lse(np32(lse), rl, what, LSE_ATOL_F32)
    else:
        for b in range(w.B):
            check_bf16(np32(o[b]), ro[b], f"{what} seq {b}")
        check_lse(np32(lse), rl, what, LSE_ATOL_BF16)


@pytest.mark.parametrize("name", ["decode_small_f32", "decode_llama70b_32k", "decode_ragged_b4"])
def test_decode_fused_workload(name):
    """The three decode workloads at full size: bitwise equal to the two
    launches, within tolerance of the oracle, three calls in a row on one
    workspace."""
    w = inputs.WORKLOADS[name]
    banner(name, "gqa_attn_decode_fused", w.lens)
    x = inputs.make_decode(w, device=DEV)
    ref_o, ref_l, outs = _pair(x, w, reps=3)
    for i, (o, lse) in enumerate(outs):
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), f"{name} call {i}"
    _check_oracle(outs[0][0], outs[0][1], x, w, name)


SHAPES = [
    # (B, H_q, H_kv, lens, kv_cap, dtype, chunk): single-split heads, ragged
    # batches whose short sequences have fewer splits than the launch, G = 1
    # and 16, 2-8 load rounds of the merge (128-key splits over 32K keys).
    (1, 8, 1, (1,), 1, "bf16", 0),
    (3, 8, 8, (127, 128, 1000), 1000, "bf16", 256),
    (4, 64, 8, (1, 700, 5000, 33), 5000, "bf16", 0),
    (2, 16, 1, (300, 17), 300, "bf16", 128),
    (1, 64, 8, (32768,), 32768, "bf16", 128),
    (2, 8, 4, (1, 700), 701, "f32", 0),
    (1, 16, 2, (5000,), 5000, "f32", 0),
]


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: f"B{c[0]}_Hq{c[1]}_Hkv{c[2]}_{c[5]}_c{c[6]}")
def test_decode_fused_shapes(case):
    B, H_q, H_kv, lens, cap, dtype, chunk = case
    w = inputs.Workload("t", "decode", B=B, H_q=H_q, H_kv=H_kv, d=128, dtype=dtype,
                        lens=lens, kv_cap=cap)
    banner("decode_fused_shapes", case)
    x = inputs.make_decode(w, device=DEV, seed=1300 + SHAPES.index(case))
    ref_o, ref_l, outs = _pair(x, w, chunk=chunk, reps=2)
    for i, (o, lse) in enumerate(outs):
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), f"{case} call {i}"
    _check_oracle(outs[0][0], outs[0][1], x, w, str(case))


def test_decode_fused_counters_return_to_zero_and_mix_with_two_launches():
    """One zeroed workspace shared by fused and two-launch calls of different
    sizes, alternating: the counter region is zero after every fused call
    and each result is bit-identical to a fresh two-launch call."""
    big = inputs.Workload("t", "decode", B=2, H_q=64, H_kv=8, d=128, dtype="bf16",
                          lens=(9000, 20000), kv_cap=20000)
    small = inputs.Workload("t", "decode", B=1, H_q=64, H_kv=8, d=128, dtype="bf16",
                            lens=(700,), kv_cap=700)
    banner("decode_fused_counters")
    xb = inputs.make_decode(big, device=DEV, seed=1401)
    xs = inputs.make_decode(small, device=DEV, seed=1402)
    need = gq.decode_workspace_bytes(2, 64, 8, 128, 20000)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    cnt_bytes = 64 << 10       # the arrival counters: the workspace's first 64 KiB
    for it, (x, w) in enumerate([(xb, big), (xs, small), (xb, big), (xs, small)]):
        kw = dict(max_kv_len=max(w.lens), scale=w.scale, return_lse=True)
        ref = gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], **kw)
        got = gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], workspace=ws, phase="fused", **kw)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), f"step {it}"
        assert int(ws[:cnt_bytes].to(torch.int32).abs().sum()) == 0, f"counters left set, step {it}"
        # A two-launch call on the same workspace leaves the counters alone.
        gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], workspace=ws, **kw)
    _check_oracle(got[0], got[1], xs, small, "decode_fused small")
