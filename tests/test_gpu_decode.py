"""Decode parity on the GPU: the HIP path through the C ABI vs the fp64 oracle."""

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


def _oracle(x, w):
    return oracle.decode(np32(x["q"]), np32(x["k"]), np32(x["v"]),
                         x["kv_lens"].cpu().numpy(), w.scale)


def _run(x, w, chunk=0):
    o, lse = gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], max_kv_len=max(w.lens),
                       scale=w.scale, chunk_tokens=chunk, return_lse=True)
    torch.cuda.synchronize()
    return o, lse


def _check(o, lse, ref_o, ref_lse, w, what):
    if w.dtype == "f32":
        check_f32(np32(o), ref_o, what)
        check_lse(np32(lse), ref_lse, what, LSE_ATOL_F32)
    else:
        for b in range(w.B):        # relative L2 per sequence
            check_bf16(np32(o[b]), ref_o[b], f"{what} seq {b}")
        check_lse(np32(lse), ref_lse, what, LSE_ATOL_BF16)


@pytest.mark.parametrize("name", ["decode_small_f32", "decode_llama70b_32k", "decode_ragged_b4"])
def test_decode_workload(name):
    """The three decode workloads at full size, automatic split (the bench's launch)."""
    w = inputs.WORKLOADS[name]
    banner(name, "gqa_attn_decode", f"B={w.B} H_q={w.H_q} H_kv={w.H_kv} lens={w.lens}")
    x = inputs.make_decode(w, device=DEV)
    o, lse = _run(x, w)
    ref_o, ref_lse = _oracle(x, w)
    _check(o, lse, ref_o, ref_lse, w, name)


SMALL = [
    # (B, H_q, H_kv, lens, kv_cap, dtype, chunk)
    (1, 8, 1, (1,), 1, "bf16", 0),
    (1, 8, 1, (5,), 40, "bf16", 0),
    (2, 8, 2, (31, 33), 64, "bf16", 128),
    (1, 16, 1, (129,), 129, "bf16", 128),
    (3, 8, 8, (127, 128, 1000), 1000, "bf16", 256),
    (2, 4, 2, (300, 17), 300, "bf16", 128),
    (1, 64, 8, (4097,), 4100, "bf16", 0),
    (2, 8, 4, (1, 700), 701, "f32", 0),
    (1, 16, 2, (513,), 513, "f32", 0),
    # fp32 split kernel: 1, 3 and 4 query slots per thread (G = 1, 12, 16)
    (1, 3, 3, (100,), 100, "f32", 0),
    (1, 12, 1, (200,), 200, "f32", 0),
    (2, 32, 2, (65, 130), 130, "f32", 0),
    # fp32 with 79 splits: the combine's second load round
    (1, 8, 1, (5000,), 5000, "f32", 0),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}_Hq{c[1]}_Hkv{c[2]}_L{c[3]}_{c[5]}_c{c[6]}")
def test_decode_shapes(case):
    """Several tiles plus a ragged tail, G in {1,2,4,8,12,16}, NaN-padded caches."""
    B, H_q, H_kv, lens, cap, dt, chunk = case
    w = inputs.Workload("t", "decode", B=B, H_q=H_q, H_kv=H_kv, d=128, dtype=dt, lens=lens,
                        kv_cap=cap)
    banner("decode_shapes", case)
    x = inputs.make_decode(w, device=DEV, seed=1000 + SMALL.index(case))
    o, lse = _run(x, w, chunk)
    ref_o, ref_lse = _oracle(x, w)
    _check(o, lse, ref_o, ref_lse, w, f"shapes {case}")


def test_decode_single_key_is_v0():
    """One valid key: O = V[0] exactly (p = l = 1), so bitwise equal."""
    w = inputs.Workload("t", "decode", B=2, H_q=16, H_kv=2, d=128, dtype="bf16", lens=(1, 1),
                        kv_cap=64)
    banner("decode_single_key")
    x = inputs.make_decode(w, device=DEV, seed=7)
    o, _ = _run(x, w)
    G = 8
    for h in range(16):
        assert torch.equal(o[:, h], x["v"][:, h // G, 0]), f"head {h}"


def test_decode_split_invariance_and_determinism():
    """Any split size reaches the oracle; the same split is bitwise repeatable.  128-key
    splits of 9000 keys give 71 partials per row: the combine's second load round."""
    w = inputs.Workload("t", "decode", B=2, H_q=64, H_kv=8, d=128, dtype="bf16",
                        lens=(9000, 3001), kv_cap=9000)
    banner("decode_split_invariance")
    x = inputs.make_decode(w, device=DEV, seed=11)
    ref_o, ref_lse = _oracle(x, w)
    outs = {}
    for chunk in (128, 384, 1024, 0):
        o, lse = _run(x, w, chunk)
        _check(o, lse, ref_o, ref_lse, w, f"chunk {chunk}")
        o2, lse2 = _run(x, w, chunk)
        assert torch.equal(o, o2) and torch.equal(lse, lse2), f"chunk {chunk} not deterministic"
        outs[chunk] = o


def test_decode_permutation_invariance():
    """Jointly permuting (k, v) pairs keeps the decode output (within tolerance)."""
    w = inputs.Workload("t", "decode", B=1, H_q=64, H_kv=8, d=128, dtype="bf16", lens=(2048,),
                        kv_cap=2048)
    banner("decode_permutation")
    x = inputs.make_decode(w, device=DEV, seed=12)
    perm = torch.randperm(2048, generator=torch.Generator().manual_seed(3)).to(DEV)
    xp = dict(x, k=x["k"][:, :, perm].contiguous(), v=x["v"][:, :, perm].contiguous())
    o, lse = _run(x, w)
    op, lsep = _run(xp, w)
    ref_o, ref_lse = _oracle(x, w)
    _check(op, lsep, ref_o, ref_lse, w, "permuted")
    _check(o, lse, ref_o, ref_lse, w, "original")


def test_decode_zero_query_is_mean():
    """Q = 0: uniform weights, O = mean of the valid V rows, lse = ln(L)."""
    w = inputs.Workload("t", "decode", B=1, H_q=8, H_kv=1, d=128, dtype="bf16", lens=(999,),
                        kv_cap=1024)
    banner("decode_zero_query")
    x = inputs.make_decode(w, device=DEV, seed=13)
    x["q"].zero_()
    o, lse = _run(x, w)
    mean = np32(x["v"][0, 0, :999]).astype(np.float64).mean(axis=0)
    for h in range(8):
        check_bf16(np32(o[0, h]), mean, f"mean head {h}", rel_l2=True)
    check_lse(np32(lse), np.full((1, 8), np.log(999.0)), "zero-q lse", LSE_ATOL_BF16)


def test_decode_workspace_reuse_and_stream():
    """One caller-owned workspace, filled with garbage first, reused across
    calls of different shapes on a side stream."""
    banner("decode_workspace_reuse")
    need = gq.decode_workspace_bytes(2, 32, 4, 128, 3000, 0, gq.DTYPE_BF16)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()
    for lens, H_q, H_kv in (((3000, 1200), 32, 4), ((700, 2999), 16, 2), ((3000, 1), 32, 4)):
        w = inputs.Workload("t", "decode", B=2, H_q=H_q, H_kv=H_kv, d=128, dtype="bf16",
                            lens=lens, kv_cap=3000)
        x = inputs.make_decode(w, device=DEV, seed=14 + H_q)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            o = gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], scale=w.scale, workspace=ws,
                          stream=s)
        s.synchronize()
        ref_o, _ = _oracle(x, w)
        for b in range(2):
            check_bf16(np32(o[b]), ref_o[b], f"ws reuse {lens} seq {b}")


def test_decode_alternating_inputs_bitwise():
    """Back-to-back calls alternating between four inputs on one workspace:
    every output equals its own first result bitwise (no stale partials)."""
    w = inputs.WORKLOADS["decode_llama70b_32k"]
    banner("decode_alternating", w.name)
    xs = [inputs.make_decode(w, device=DEV, seed=40 + i) for i in range(4)]
    need = gq.decode_workspace_bytes(1, 64, 8, 128, 32768, 0, gq.DTYPE_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    refs = [gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], scale=w.scale, workspace=ws).clone()
            for x in xs]
    outs = [torch.empty_like(refs[0]) for _ in range(64)]
    for i in range(64):
        x = xs[i % 4]
        gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], scale=w.scale, out=outs[i], workspace=ws)
    torch.cuda.synchronize()
    for i in range(64):
        assert torch.equal(outs[i], refs[i % 4]), f"call {i} differs"


def test_decode_phases_equal_one_call():
    """gqa_attn_decode_partial then _combine on one stream is gqa_attn_decode."""
    w = inputs.Workload("t", "decode", B=3, H_q=64, H_kv=8, d=128, dtype="bf16",
                        lens=(4000, 70, 2500), kv_cap=4096)
    banner("decode_phases")
    x = inputs.make_decode(w, device=DEV, seed=31)
    ws = torch.empty(gq.decode_workspace_bytes(3, 64, 8, 128, 4000, 0, gq.DTYPE_BF16),
                     dtype=torch.uint8, device=DEV)
    one, l1 = gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], max_kv_len=4000, scale=w.scale,
                        return_lse=True, workspace=ws)
    two = torch.empty_like(one)
    l2 = torch.empty_like(l1)
    gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], max_kv_len=4000, scale=w.scale,
              return_lse=True, out=two, lse=l2, workspace=ws, phase="partial")
    gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], max_kv_len=4000, scale=w.scale,
              return_lse=True, out=two, lse=l2, workspace=ws, phase="combine")
    torch.cuda.synchronize()
    assert torch.equal(one, two) and torch.equal(l1, l2)


@pytest.mark.parametrize("chunk", [0, 128])
def test_decode_max_jump(chunk):
    """Keys of one later stretch scaled by 40 (and a few more by 25): the
    running max jumps inside a split and between splits; every element
    against the oracle."""
    w = inputs.Workload("t", "decode", B=2, H_q=16, H_kv=2, d=128, dtype="bf16",
                        lens=(5000, 3100), kv_cap=5000)
    banner("decode_max_jump", chunk)
    x = inputs.make_decode(w, device=DEV, seed=17)
    x["k"][:, :, 3000:3100] *= 40.0
    x["k"][:, :, 4500:4510] *= 25.0
    o, lse = _run(x, w, chunk)
    ref_o, ref_lse = _oracle(x, w)
    _check(o, lse, ref_o, ref_lse, w, f"max jump chunk={chunk}")
