"""Paged-cache varlen prefill parity on the GPU: gqa_attn_prefill_paged through
the C ABI vs the fp64 oracle, and bitwise against gqa_attn_prefill_varlen on
the contiguous cache the pages were scattered from (the same tiles, the same
arithmetic).  Unused pages, table entries past a sequence's pages and rows of
a last page past its length are NaN, so reading any of them poisons the
output."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_ATOL_BF16, banner, check_bf16, check_lse, np32
from gqa_flashattention_amd import binding as gq
from gqa_flashattention_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _workload(H_q, H_kv, q_lens, lens, cap, page, causal=True):
    return inputs.Workload("t", "prefill_paged", B=len(q_lens), H_q=H_q, H_kv=H_kv, d=128,
                           dtype="bf16", q_lens=tuple(q_lens), lens=tuple(lens), kv_cap=cap,
                           causal=causal, page_size=page)


def _run_paged(x, w, **kw):
    o, lse = gq.prefill_paged(x["q"], x["k_pages"], x["v_pages"], x["block_table"],
                              x["cu_seqlens_q"], x["kv_lens"], max_seqlen_q=max(w.q_lens),
                              max_kv_len=max(w.lens), causal=w.causal, scale=w.scale,
                              return_lse=True, **kw)
    torch.cuda.synchronize()
    return o, lse


def _run_contiguous(x, w):
    o, lse = gq.prefill_varlen(x["q"], x["k"], x["v"], x["cu_seqlens_q"], x["kv_lens"],
                               max_seqlen_q=max(w.q_lens), max_kv_len=max(w.lens),
                               causal=w.causal, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    return o, lse


SHAPES = [
    # (H_q, H_kv, q_lens, kv_lens, kv_cap, page, causal)
    (8, 1, (1, 300, 0, 64), (1, 300, 5, 1000), 1000, 16, True),
    (64, 8, (100, 513, 7), (100, 2000, 7), 2048, 16, True),     # Llama geometry, ragged tails
    (64, 8, (100, 513, 7), (100, 2000, 7), 2048, 32, True),
    (16, 2, (77, 250), (1000, 700), 1000, 64, False),           # non-causal
    (16, 8, (150, 1, 33), (150, 4097, 33), 4100, 128, True),    # G = 2
    (32, 2, (70, 129), (70, 300), 300, 1024, True),             # G = 16; pages longer than caches
    (8, 8, (257, 64, 65), (257, 1000, 65), 1000, 256, True),    # G = 1
]


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: f"Hq{c[0]}_Hkv{c[1]}_P{c[5]}_"
                                                      f"{'c' if c[6] else 'nc'}_L{'-'.join(map(str, c[3]))}")
def test_prefill_paged_shapes(case):
    """Every element against the oracle over the pages, and bitwise against
    the contiguous-cache launch."""
    H_q, H_kv, q_lens, lens, cap, page, causal = case
    w = _workload(H_q, H_kv, q_lens, lens, cap, page, causal)
    banner("prefill_paged_shapes", case)
    x = inputs.make_prefill_paged(w, page, device=DEV, seed=3600 + SHAPES.index(case))
    o, lse = _run_paged(x, w)
    oc, lc = _run_contiguous(x, w)
    assert torch.equal(o, oc) and torch.equal(lse, lc)
    ro, rl = oracle.prefill_paged(np32(x["q"]), np32(x["k_pages"]), np32(x["v_pages"]),
                                  x["block_table"].cpu().numpy(), x["cu_seqlens_q"].cpu().numpy(),
                                  np.array(lens), page, w.scale, causal=causal)
    cu = x["cu_seqlens_q"].cpu().tolist()
    for b in range(w.B):
        if cu[b + 1] > cu[b]:
            check_bf16(np32(o[cu[b]:cu[b + 1]]), ro[cu[b]:cu[b + 1]], f"{case} seq {b}")
            check_lse(np32(lse[cu[b]:cu[b + 1]]), rl[cu[b]:cu[b + 1]], f"{case} seq {b}",
                      LSE_ATOL_BF16)


def test_prefill_paged_workload():
    """The chunked-prefill batch over 16-position pages at full size (the
    bench's launch): finite, bitwise equal to the contiguous-cache launch
    (whose every chunk the varlen tests check against the oracle), and the
    oracle on seeded (head, row) pairs of the 64K-context chunk."""
    name = "prefill_paged_llama70b_b8_p16"
    w = inputs.WORKLOADS[name]
    banner(name, "gqa_attn_prefill_paged", f"page={w.page_size}")
    x = inputs.make_prefill_paged(w, w.page_size, device=DEV)
    o, lse = _run_paged(x, w)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    oc, lc = _run_contiguous(x, w)
    assert torch.equal(o, oc) and torch.equal(lse, lc)
    b = 4                                   # 512 tokens over 65536 positions
    cu = x["cu_seqlens_q"].cpu().tolist()
    sq, L = w.q_lens[b], w.lens[b]
    rows = np.array(inputs.sample_rows(sq, 24, inputs.SEEDS[name]))
    qb = np.transpose(np32(x["q"][cu[b]:cu[b + 1]]), (1, 0, 2))[None]
    k32, v32 = np32(x["k"][b:b + 1]), np32(x["v"][b:b + 1])
    for h in (0, 37, 63):
        ro, rl = oracle.prefill(qb, k32, v32, L, w.scale, causal=True, causal_offset=L - sq,
                                rows=rows, heads=[h])
        idx = torch.as_tensor(cu[b] + rows, device=DEV)
        check_bf16(np32(o[idx, h]), ro[0, 0], f"{name} head {h}")
        check_lse(np32(lse[idx, h]), rl[0, 0], f"{name} head {h}", LSE_ATOL_BF16)


def test_prefill_paged_bad_table_entries_stay_in_pool():
    """Table entries outside [0, num_pages) are clamped into the pool: the
    call completes and reads only pool pages (the result for that sequence is
    meaningless; the other sequence is unaffected and exact)."""
    w = _workload(16, 2, (40, 30), (300, 200), 320, 16)
    banner("prefill_paged_bad_entries")
    x = inputs.make_prefill_paged(w, 16, device=DEV, seed=3700)
    x["block_table"][1, 3] = 1 << 30
    x["block_table"][1, 5] = -7
    o, _ = _run_paged(x, w)
    oc, _ = _run_contiguous(x, w)
    assert torch.equal(o[:40], oc[:40])
