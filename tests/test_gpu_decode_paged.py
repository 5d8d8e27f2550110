"""Paged-cache decode on the GPU: gqa_attn_decode_paged through the C ABI vs
the fp64 oracle, and bitwise against the same call on the contiguous cache
(the kernels fold the same blocks in the same order)."""

import pytest
import torch

import oracle
from gpu_util import LSE_ATOL_BF16, banner, check_bf16, check_lse, np32
from gqa_flashattention_amd import binding as gq
from gqa_flashattention_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check(o, lse, x, w, page, what):
    ref_o, ref_lse = oracle.decode_paged(np32(x["q"]), np32(x["k_pages"]), np32(x["v_pages"]),
                                         x["block_table"].cpu().numpy(),
                                         x["kv_lens"].cpu().numpy(), page, w.scale)
    for b in range(w.B):
        check_bf16(np32(o[b]), ref_o[b], f"{what} seq {b}")
    check_lse(np32(lse), ref_lse, what, LSE_ATOL_BF16)


CASES = [
    # (B, H_q, H_kv, T_q, lens, kv_cap, page, chunk)
    (1, 8, 1, 1, (1,), 16, 16, 0),
    (3, 64, 8, 1, (1000, 37, 4097), 4100, 16, 0),
    (2, 64, 8, 1, (5000, 129), 5000, 64, 0),
    (2, 16, 2, 2, (700, 2), 768, 32, 128),
    (1, 64, 8, 2, (3000,), 3000, 128, 0),
    (2, 64, 8, 4, (2049, 64), 2100, 64, 0),           # multi-token kernel, 32 rows
    (2, 32, 4, 8, (1500, 9), 1536, 16, 256),          # 64 rows, pages of 16
    (1, 64, 8, 16, (4097,), 4100, 1024, 0),           # 128 rows, large pages
    (2, 64, 8, 16, (777, 3333), 3584, 32, 0),
]


@pytest.mark.parametrize("case", CASES,
                         ids=lambda c: f"B{c[0]}_Hq{c[1]}_T{c[3]}_L{c[4]}_p{c[6]}_c{c[7]}")
def test_decode_paged_shapes(case):
    B, H_q, H_kv, T_q, lens, cap, page, chunk = case
    w = inputs.Workload("t", "decode_multi", B=B, H_q=H_q, H_kv=H_kv, d=128, dtype="bf16",
                        lens=lens, kv_cap=cap, T_q=T_q)
    banner("decode_paged", case)
    x = inputs.make_decode_paged(w, page, device=DEV, seed=3000 + CASES.index(case))
    o, lse = gq.decode_paged(x["q"], x["k_pages"], x["v_pages"], x["block_table"], x["kv_lens"],
                             max_kv_len=max(lens), scale=w.scale, chunk_tokens=chunk,
                             return_lse=True)
    torch.cuda.synchronize()
    _check(o, lse, x, w, page, f"paged {case}")
    # The contiguous cache with the split the paged call used.
    c = gq.decode_paged_split_tokens(B, H_q, H_kv, T_q, page, max(lens), chunk)
    oc, lc = gq.decode_multi(x["q"], x["k"], x["v"], x["kv_lens"], max_kv_len=max(lens),
                             scale=w.scale, chunk_tokens=c, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(lse, lc), "paged differs from contiguous"


def test_decode_paged_workload():
    """The paged 32K workload at full size (the bench's launch)."""
    w = inputs.WORKLOADS["decode_paged_llama70b_32k_p64"]
    banner(w.name)
    x = inputs.make_decode_paged(w, w.page_size, device=DEV)
    o, lse = gq.decode_paged(x["q"], x["k_pages"], x["v_pages"], x["block_table"], x["kv_lens"],
                             max_kv_len=w.max_kv_len, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    _check(o, lse, x, w, w.page_size, w.name)
