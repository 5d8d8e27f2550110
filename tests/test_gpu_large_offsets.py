"""64-bit addressing on the GPU: every entry point reads K/V (and reads Q,
writes O) at byte offsets past 2^31 of its tensors, compared with the fp64
oracle.

The K/V cache is one allocation holding all sequences' contiguous blocks
(the per-sequence placement of contiguous blocks, ADR-0060@5a76ed4 §2.1 "KV
cache allocation"); with long capacities or large batches the later blocks
start gigabytes into it, so any 32-bit byte offset in a kernel's addressing
would wrap and read the wrong rows.  Each case states the smallest offset it
touches.  Padding is NaN, so a wrapped read of unused capacity poisons the
output instead of passing silently."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_ATOL_BF16, banner, check_bf16, check_lse, np32
from gqa_flashattention_amd import binding as gq
from gqa_flashattention_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
TWO_GIB = 1 << 31
ROW_BYTES = 128 * 2     # one bf16 row of d = 128


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def long_cache():
    """Decode inputs with a 2^20-position capacity: sequence 1's K/V blocks
    start 2 GiB into the cache tensors (up to 3.75 GiB for KV head 7)."""
    w = inputs.Workload("t", "decode", B=2, H_q=64, H_kv=8, d=128, dtype="bf16",
                        lens=(777, 300000), kv_cap=1 << 20)
    banner("large_offsets decode cache", w.kv_cap)
    x = inputs.make_decode(w, device=DEV, seed=31)
    assert 1 * w.H_kv * w.kv_cap * ROW_BYTES >= TWO_GIB
    yield w, x
    del x
    _free()


def _oracle_decode_per_sequence(q, k, v, lens, scale, fn):
    outs, lses = [], []
    for b, L in enumerate(lens):
        ro, rl = fn(np32(q[b:b + 1]), np32(k[b:b + 1, :, :L]), np32(v[b:b + 1, :, :L]),
                    np.array([L]), scale)
        outs.append(ro)
        lses.append(rl)
    return np.concatenate(outs), np.concatenate(lses)


def test_decode_kv_past_2gib(long_cache):
    w, x = long_cache
    o, lse = gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], max_kv_len=max(w.lens),
                       scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = _oracle_decode_per_sequence(x["q"], x["k"], x["v"], w.lens, w.scale, oracle.decode)
    for b in range(w.B):
        check_bf16(np32(o[b]), ro[b], f"decode seq {b}")
    check_lse(np32(lse), rl, "decode", LSE_ATOL_BF16)


def test_decode_multi_kv_past_2gib(long_cache):
    """T_q = 4 (32 folded rows: the multi-token kernel) on the same cache."""
    w, x = long_cache
    q = inputs.randn((w.B, w.H_q, 4, w.d), torch.bfloat16, DEV, 32, 3)
    o, lse = gq.decode_multi(q, x["k"], x["v"], x["kv_lens"], max_kv_len=max(w.lens),
                             scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = _oracle_decode_per_sequence(q, x["k"], x["v"], w.lens, w.scale,
                                         oracle.decode_multi)
    for b in range(w.B):
        check_bf16(np32(o[b]), ro[b], f"decode_multi seq {b}")
    check_lse(np32(lse), rl, "decode_multi", LSE_ATOL_BF16)


def test_prefill_q_o_and_kv_past_2gib():
    """33 sequences of 4096 causal positions: sequence 32's Q and O rows
    start 2 GiB into q and o, and its K/V blocks (32768-position capacity)
    2 GiB into k and v.  Sampled rows of sequence 32 (all 64 heads, the
    last row included) and of sequence 0 against the oracle."""
    w = inputs.Workload("t", "prefill", B=33, H_q=64, H_kv=8, d=128, dtype="bf16", S_q=4096,
                        S_kv=4096, causal=True, offset=0)
    banner("large_offsets prefill", w.B, w.S_q)
    x = inputs.make_prefill(w, device=DEV, seed=33, kv_cap=32768)
    assert 32 * w.H_q * w.S_q * ROW_BYTES >= TWO_GIB
    assert 32 * w.H_kv * 32768 * ROW_BYTES >= TWO_GIB
    o, lse = gq.prefill(x["q"], x["k"], x["v"], S_kv=w.S_kv, causal=True, scale=w.scale,
                        return_lse=True)
    torch.cuda.synchronize()
    rows = np.asarray(inputs.sample_rows(w.S_q, 192, 34))
    for b in (0, 32):
        ro, rl = oracle.prefill(np32(x["q"][b:b + 1]), np32(x["k"][b:b + 1, :, :w.S_kv]),
                                np32(x["v"][b:b + 1, :, :w.S_kv]), w.S_kv, w.scale,
                                causal=True, rows=rows)
        got = np32(o[b][:, rows])
        for h in range(w.H_q):
            check_bf16(got[h], ro[0, h], f"prefill seq {b} head {h}")
        check_lse(np32(lse[b][:, rows]), rl[0], f"prefill seq {b}", LSE_ATOL_BF16)
    del x, o, lse
    _free()


def _paged_pool_past_2gib(L, page, seed):
    """A contiguous cache of one sequence of L positions and a pool of
    page-size pages whose used pages all sit past byte offset 2^31 of the
    pool (in a seeded random order); the other pages are NaN."""
    page_bytes = 8 * page * ROW_BYTES
    first = TWO_GIB // page_bytes
    n = (L + page - 1) // page
    num_pages = first + n + 2
    k = inputs.randn((1, 8, n * page, 128), torch.bfloat16, DEV, seed, 1)
    v = inputs.randn((1, 8, n * page, 128), torch.bfloat16, DEV, seed, 2)
    k[:, :, L:] = float("nan")
    v[:, :, L:] = float("nan")
    g = torch.Generator().manual_seed(seed)
    phys = (first + torch.randperm(n, generator=g)).to(DEV)
    pools = []
    for src in (k, v):
        pool = torch.full((num_pages, 8, page, 128), float("nan"), dtype=torch.bfloat16,
                          device=DEV)
        pool[phys] = src[0].reshape(8, n, page, 128).transpose(0, 1)
        pools.append(pool)
    table = phys.to(torch.int32).reshape(1, n).contiguous()
    assert int(phys.min()) * page_bytes >= TWO_GIB
    return k, v, pools[0], pools[1], table


def test_decode_paged_pages_past_2gib():
    L, page = 20000, 64
    banner("large_offsets decode_paged", L, page)
    k, v, kp, vp, table = _paged_pool_past_2gib(L, page, 35)
    q = inputs.randn((1, 64, 1, 128), torch.bfloat16, DEV, 35, 0)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    o, lse = gq.decode_paged(q, kp, vp, table, lens, max_kv_len=L, scale=128 ** -0.5,
                             return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_multi(np32(q), np32(k[:, :, :L]), np32(v[:, :, :L]), np.array([L]),
                                 128 ** -0.5)
    check_bf16(np32(o[0]), ro[0], "decode_paged")
    check_lse(np32(lse), rl, "decode_paged", LSE_ATOL_BF16)
    del k, v, kp, vp
    _free()


def test_prefill_paged_pages_past_2gib():
    """A 300-token chunk at the end of a 20000-position sequence whose pages
    all lie past 2 GiB of the pool: every element against the oracle, and
    bitwise against the contiguous-cache varlen launch."""
    L, page, S_q = 20000, 64, 300
    banner("large_offsets prefill_paged", L, page, S_q)
    k, v, kp, vp, table = _paged_pool_past_2gib(L, page, 36)
    q = inputs.randn((S_q, 64, 128), torch.bfloat16, DEV, 36, 0)
    cu = torch.tensor([0, S_q], dtype=torch.int32, device=DEV)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    kw = dict(max_seqlen_q=S_q, max_kv_len=L, causal=True, scale=128 ** -0.5, return_lse=True)
    o, lse = gq.prefill_paged(q, kp, vp, table, cu, lens, **kw)
    oc, lc = gq.prefill_varlen(q, k, v, cu, lens, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(lse, lc)
    ro, rl = oracle.prefill_varlen(np32(q), np32(k[:, :, :L]), np32(v[:, :, :L]),
                                   np.array([0, S_q]), np.array([L]), 128 ** -0.5)
    check_bf16(np32(o), ro, "prefill_paged")
    check_lse(np32(lse), rl, "prefill_paged", LSE_ATOL_BF16)
    del k, v, kp, vp
    _free()
