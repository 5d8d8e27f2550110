"""Stitching (gqa_attn_merge) on the GPU against the fp64 oracle: attention
over keys split into chunks, each chunk computed by the library, merged by
the library, equals attention over all keys."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_ATOL_BF16, LSE_ATOL_F32, banner, check_bf16, check_f32, check_lse, np32
from gqa_flashattention_amd import binding as gq
from gqa_flashattention_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("dtype,cut", [("bf16", 1), ("bf16", 2048), ("bf16", 4999), ("f32", 300)])
def test_merge_two_decode_chunks(dtype, cut):
    """Decode over keys [0, cut) and [cut, L) as two library calls, stitched,
    against the oracle over all L keys and against the oracle's own stitch
    of the two GPU chunk results."""
    L = 5000
    H_q, H_kv = (64, 8) if dtype == "bf16" else (8, 1)
    w = inputs.Workload("t", "decode", B=2, H_q=H_q, H_kv=H_kv, d=128, dtype=dtype,
                        lens=(L, L), kv_cap=L)
    banner("merge_decode_chunks", dtype, cut)
    x = inputs.make_decode(w, device=DEV, seed=61)
    ka, va = x["k"][:, :, :cut].contiguous(), x["v"][:, :, :cut].contiguous()
    kb, vb = x["k"][:, :, cut:].contiguous(), x["v"][:, :, cut:].contiguous()
    la_len = torch.full((2,), cut, dtype=torch.int32, device=DEV)
    lb_len = torch.full((2,), L - cut, dtype=torch.int32, device=DEV)
    oa, lsa = gq.decode(x["q"], ka, va, la_len, max_kv_len=cut, scale=w.scale, return_lse=True)
    ob, lsb = gq.decode(x["q"], kb, vb, lb_len, max_kv_len=L - cut, scale=w.scale, return_lse=True)
    o, lse = gq.merge(oa, lsa, ob, lsb, return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.decode(np32(x["q"]), np32(x["k"]), np32(x["v"]), np.array([L, L]), w.scale)
    if dtype == "bf16":
        for b in range(2):
            check_bf16(np32(o[b]), ref_o[b], f"stitched seq {b}")
        check_lse(np32(lse), ref_l, "stitched lse", LSE_ATOL_BF16)
    else:
        check_f32(np32(o), ref_o, "stitched f32")
        check_lse(np32(lse), ref_l, "stitched lse f32", LSE_ATOL_F32)
    # The kernel's merge against the oracle's merge of the same two inputs.
    so, sl = oracle.merge_normalized(np32(oa), np32(lsa), np32(ob), np32(lsb))
    tol = 2.0 ** -8 if dtype == "bf16" else 1e-6
    assert np.max(np.abs(np32(o) - so) - tol * np.abs(so)) <= 1e-6
    assert np.max(np.abs(np32(lse) - sl)) <= 1e-5


def test_merge_prefix_and_causal_chunk():
    """A chunk of S_q queries after `off` cached keys: non-causal attention
    over the prefix plus causal attention over the chunk's own keys,
    stitched, equals the causal prefill with offset `off`."""
    off, S_q = 1000, 300
    S_kv = off + S_q
    w = inputs.Workload("t", "prefill", B=1, H_q=16, H_kv=2, d=128, dtype="bf16", S_q=S_q,
                        S_kv=S_kv, causal=True, offset=off)
    banner("merge_prefix_chunk")
    x = inputs.make_prefill(w, device=DEV, seed=62)
    kp, vp = x["k"][:, :, :off].contiguous(), x["v"][:, :, :off].contiguous()
    kc, vc = x["k"][:, :, off:].contiguous(), x["v"][:, :, off:].contiguous()
    o1, l1 = gq.prefill(x["q"], kp, vp, S_kv=off, causal=False, scale=w.scale, return_lse=True)
    o2, l2 = gq.prefill(x["q"], kc, vc, S_kv=S_q, causal=True, causal_offset=0, scale=w.scale,
                        return_lse=True)
    o, lse = gq.merge(o1, l1, o2, l2, return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.prefill(np32(x["q"]), np32(x["k"]), np32(x["v"]), S_kv, w.scale,
                                  causal=True, causal_offset=off)
    check_bf16(np32(o[0]), ref_o[0], "prefix + chunk")
    check_lse(np32(lse), ref_l, "prefix + chunk lse", LSE_ATOL_BF16)


def test_merge_empty_sides_and_aliasing():
    """lse = -inf on one side gives the other side exactly (its O may be
    NaN); both empty gives O = 0 and lse = -inf; output written in place
    over input A."""
    banner("merge_empty_and_alias")
    rows = 1000
    g = torch.Generator(device=DEV).manual_seed(63)
    oa = torch.randn(rows, 128, device=DEV, generator=g).to(torch.bfloat16)
    ob = torch.randn(rows, 128, device=DEV, generator=g).to(torch.bfloat16)
    la = torch.randn(rows, device=DEV, generator=g) * 3
    lb = torch.randn(rows, device=DEV, generator=g) * 3
    lb[::3] = float("-inf")
    ob[::3] = float("nan")
    la[1::3] = float("-inf")
    oa[1::3] = float("nan")
    la[2::9] = float("-inf")
    lb[2::9] = float("-inf")
    exp_o, exp_l = oracle.merge_normalized(np32(oa), np32(la), np32(ob), np32(lb))
    oa0, ob0, la0, lb0 = oa.clone(), ob.clone(), la.clone(), lb.clone()
    o, lse = gq.merge(oa, la, ob, lb, out=oa, lse_out=la, return_lse=True)   # in place over A
    torch.cuda.synchronize()
    assert o.data_ptr() == oa.data_ptr()
    assert torch.equal(o[::3], oa0[::3]) and torch.equal(lse[::3], la0[::3])     # B empty
    assert torch.equal(o[1::3], ob0[1::3]) and torch.equal(lse[1::3], lb0[1::3])  # A empty
    both = torch.zeros(rows, dtype=torch.bool)
    both[2::9] = True
    assert torch.all(o[both] == 0) and torch.all(torch.isneginf(lse[both]))
    rest = ~both
    rest[::3] = False
    rest[1::3] = False
    got, ref = np32(o)[rest.numpy()], exp_o[rest.numpy()]
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - ref) - 2.0 ** -8 * np.abs(ref)) <= 1e-6
    assert np.max(np.abs(np32(lse)[rest.numpy()] - exp_l[rest.numpy()])) <= 1e-5
