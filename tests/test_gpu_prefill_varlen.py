"""Varlen prefill parity on the GPU: gqa_attn_prefill_varlen through the C ABI
vs the fp64 oracle (chunk b is the newest S_q_b of kv_lens[b] positions, so
its token i sees keys 0 .. kv_lens[b] - S_q_b + i), and bitwise against the
dense entry point called once per sequence."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_ATOL_BF16, banner, check_bf16, check_lse, np32
from gqa_flashattention_amd import binding as gq
from gqa_flashattention_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _workload(H_q, H_kv, q_lens, lens, cap, causal=True):
    return inputs.Workload("t", "prefill_varlen", B=len(q_lens), H_q=H_q, H_kv=H_kv, d=128,
                           dtype="bf16", q_lens=tuple(q_lens), lens=tuple(lens), kv_cap=cap,
                           causal=causal)


def _run(x, w, scale=None, **kw):
    o, lse = gq.prefill_varlen(x["q"], x["k"], x["v"], x["cu_seqlens_q"], x["kv_lens"],
                               max_seqlen_q=max(w.q_lens), max_kv_len=max(max(w.lens), 1),
                               causal=w.causal, scale=w.scale if scale is None else scale,
                               return_lse=True, **kw)
    torch.cuda.synchronize()
    return o, lse


def _check_all(x, w, o, lse, what, scale=None):
    """Every element of every chunk against the oracle."""
    ro, rl = oracle.prefill_varlen(np32(x["q"]), np32(x["k"]), np32(x["v"]),
                                   x["cu_seqlens_q"].cpu().numpy(), np.array(w.lens),
                                   w.scale if scale is None else scale, causal=w.causal)
    cu = x["cu_seqlens_q"].cpu().tolist()
    for b in range(w.B):
        if cu[b + 1] == cu[b]:
            continue
        check_bf16(np32(o[cu[b]:cu[b + 1]]), ro[cu[b]:cu[b + 1]], f"{what} seq {b}")
        check_lse(np32(lse[cu[b]:cu[b + 1]]), rl[cu[b]:cu[b + 1]], f"{what} seq {b}",
                  LSE_ATOL_BF16)


SMALL = [
    # (H_q, H_kv, q_lens, kv_lens, kv_cap, causal)
    (8, 1, (1, 300, 0, 64), (1, 300, 5, 1000), 1000, True),     # L = S_q; an empty chunk
    (64, 8, (100, 513, 7), (100, 2000, 7), 2048, True),         # Llama geometry, ragged tails
    (16, 2, (77, 250), (1000, 700), 1000, False),               # non-causal
    (16, 8, (150, 1, 33), (150, 4097, 33), 4100, True),         # G = 2; a one-token chunk
    (12, 2, (100, 5), (400, 5), 400, True),                     # G = 6: 2 heads x 4 blocks
    (32, 2, (70, 129), (70, 300), 300, True),                   # G = 16: two head groups
    (8, 8, (257, 64, 65), (257, 1000, 65), 1000, True),         # G = 1
    (64, 8, (1,), (5000,), 5000, True),                         # B = 1, a decode-like chunk
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"Hq{c[0]}_Hkv{c[1]}_q{'-'.join(map(str, c[2]))}"
                                                      f"_L{'-'.join(map(str, c[3]))}_{'c' if c[5] else 'nc'}")
def test_prefill_varlen_shapes(case):
    """Ragged chunk lengths and cache lengths in one launch, empty and
    one-token chunks, GQA group sizes 1..16, NaN past every cache length."""
    H_q, H_kv, q_lens, lens, cap, causal = case
    w = _workload(H_q, H_kv, q_lens, lens, cap, causal)
    banner("prefill_varlen_shapes", case)
    x = inputs.make_prefill_varlen(w, device=DEV, seed=3000 + SMALL.index(case))
    o, lse = _run(x, w)
    _check_all(x, w, o, lse, f"{case}")


def _dense_per_sequence(x, w, scale=None):
    """The dense entry point once per sequence (head-major copies of its
    chunk, causal_offset = L - S_q), packed back token-major."""
    cu = x["cu_seqlens_q"].cpu().tolist()
    o = torch.zeros_like(x["q"])
    lse = torch.zeros(x["q"].shape[:2], dtype=torch.float32, device=DEV)
    for b in range(w.B):
        t0, t1, L = cu[b], cu[b + 1], w.lens[b]
        if t1 == t0:
            continue
        qb = x["q"][t0:t1].transpose(0, 1).unsqueeze(0).contiguous()
        ob, lb = gq.prefill(qb, x["k"][b:b + 1], x["v"][b:b + 1], S_kv=L, causal=w.causal,
                            causal_offset=L - (t1 - t0) if w.causal else 0,
                            scale=w.scale if scale is None else scale, return_lse=True)
        o[t0:t1] = ob[0].transpose(0, 1)
        lse[t0:t1] = lb[0].transpose(0, 1)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("idx", [0, 1, 3, 4, 5])
def test_prefill_varlen_equals_dense_bitwise(idx):
    """One varlen launch equals the dense kernel run per sequence, bit for
    bit (the same tiles in the same order), and repeats bitwise."""
    H_q, H_kv, q_lens, lens, cap, causal = SMALL[idx]
    w = _workload(H_q, H_kv, q_lens, lens, cap, causal)
    banner("prefill_varlen_vs_dense", SMALL[idx])
    x = inputs.make_prefill_varlen(w, device=DEV, seed=3100 + idx)
    o, lse = _run(x, w)
    od, ld = _dense_per_sequence(x, w)
    assert torch.equal(o, od) and torch.equal(lse, ld)
    o2, lse2 = _run(x, w)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_prefill_varlen_workload_sampled():
    """The chunked-prefill batch at full size (the bench's launch): no
    non-finite output, every chunk bitwise equal to the dense kernel on it,
    and the oracle on seeded (head, row) pairs of every chunk plus its
    first and last rows on every head."""
    name = "prefill_varlen_llama70b_b8"
    w = inputs.WORKLOADS[name]
    banner(name, "gqa_attn_prefill_varlen", f"q_lens={w.q_lens} lens={w.lens}")
    x = inputs.make_prefill_varlen(w, device=DEV)
    o, lse = _run(x, w)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    od, ld = _dense_per_sequence(x, w)
    assert torch.equal(o, od) and torch.equal(lse, ld)
    cu = x["cu_seqlens_q"].cpu().tolist()
    q32, k32, v32 = np32(x["q"]), np32(x["k"]), np32(x["v"])
    got, want, got_l, want_l = [], [], [], []
    g = torch.Generator().manual_seed(inputs.SEEDS[name])
    for b in range(w.B):
        sq, L = w.q_lens[b], w.lens[b]
        rows = inputs.sample_rows(sq, min(sq, 24), inputs.SEEDS[name] + b)
        heads = torch.randint(0, w.H_q, (len(rows),), generator=g).tolist()
        by_head = {}
        for h, r in zip(heads, rows):
            by_head.setdefault(h, set()).add(r)
        for h in range(w.H_q):
            by_head.setdefault(h, set()).update({0, sq - 1})
        qb = np.transpose(q32[cu[b]:cu[b + 1]], (1, 0, 2))[None]
        for h, rs in sorted(by_head.items()):
            rs = np.array(sorted(rs))
            ro, rl = oracle.prefill(qb, k32[b:b + 1], v32[b:b + 1], L, w.scale, causal=True,
                                    causal_offset=L - sq, rows=rs, heads=[h])
            idx = torch.as_tensor(cu[b] + rs, device=DEV)
            got.append(np32(o[idx, h]))
            want.append(ro[0, 0])
            got_l.append(np32(lse[idx, h]))
            want_l.append(rl[0, 0])
    check_bf16(np.concatenate(got), np.concatenate(want), name)
    check_lse(np.concatenate(got_l), np.concatenate(want_l), name, LSE_ATOL_BF16)


def test_prefill_varlen_empty_cache_non_causal():
    """A non-causal chunk whose cache is empty sees no key: O = 0 and
    lse = -inf (the oracle's empty result); the other chunks are unaffected."""
    w = _workload(16, 2, (5, 40, 3), (300, 0, 64), 300, causal=False)
    banner("prefill_varlen_empty_cache")
    x = inputs.make_prefill_varlen(w, device=DEV, seed=3200)
    out = torch.full_like(x["q"], float("nan"))
    o, lse = _run(x, w, out=out)
    assert torch.all(o[5:45] == 0)
    assert torch.all(lse[5:45] == float("-inf"))
    ro, rl = oracle.prefill_varlen(np32(x["q"]), np32(x["k"]), np32(x["v"]),
                                   x["cu_seqlens_q"].cpu().numpy(), np.array(w.lens), w.scale,
                                   causal=False)
    assert np.all(ro[5:45] == 0) and np.all(rl[5:45] == -np.inf)
    for sl in (slice(0, 5), slice(45, 48)):
        check_bf16(np32(o[sl]), ro[sl], "empty-cache batch")
        check_lse(np32(lse[sl]), rl[sl], "empty-cache batch", LSE_ATOL_BF16)


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.3])
def test_prefill_varlen_scales(scale):
    """Negative (Q's sign flipped), zero (uniform weights) and large scales."""
    w = _workload(16, 2, (90, 17, 130), (200, 17, 1000), 1000)
    banner("prefill_varlen_scale", scale)
    x = inputs.make_prefill_varlen(w, device=DEV, seed=3300)
    o, lse = _run(x, w, scale=scale)
    _check_all(x, w, o, lse, f"scale {scale}", scale=scale)


def test_prefill_varlen_writes_every_row_and_only_its_rows():
    """Every token-packed output row is written (a NaN-filled output comes
    back finite) and a buffer with spare rows after total_q keeps them."""
    w = _workload(64, 8, (300, 1, 129), (300, 900, 2000), 2048)
    banner("prefill_varlen_rows_written")
    x = inputs.make_prefill_varlen(w, device=DEV, seed=3400)
    total = w.total_q
    big = torch.full((total + 40, w.H_q, w.d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lbig = torch.full((total + 40, w.H_q), 7.0, dtype=torch.float32, device=DEV)
    gq.prefill_varlen(x["q"], x["k"], x["v"], x["cu_seqlens_q"], x["kv_lens"],
                      max_seqlen_q=300, max_kv_len=2000, causal=True, scale=w.scale,
                      return_lse=True, out=big[:total], lse=lbig[:total])
    torch.cuda.synchronize()
    assert torch.isfinite(big[:total]).all() and torch.isfinite(lbig[:total]).all()
    assert big[total:].isnan().all() and torch.all(lbig[total:] == 7.0)
    _check_all(x, w, big[:total], lbig[:total], "rows written")


def _item_tiles(w, item, n_qblk, rows):
    """Key tiles the workgroup of work item b * n_qblk + pblk walks."""
    b, pblk = divmod(item, n_qblk)
    sq, L = w.q_lens[b], w.lens[b]
    P0 = pblk * rows
    if P0 >= sq:
        return 0
    kend = min(L, max(L - sq, 0) + P0 + rows) if w.causal else L
    return -(-kend // 64)


def test_prefill_varlen_work_list_is_sorted_permutation():
    """The pre-pass leaves every (sequence, query block) item in the
    workspace exactly once, in non-increasing tile count, whatever the
    workspace held before."""
    w = _workload(8, 1, (2048, 512, 37, 0, 1), (2048, 20000, 300, 9, 40), 20000)
    banner("prefill_varlen_work_list")
    x = inputs.make_prefill_varlen(w, device=DEV, seed=3500)
    need = gq.prefill_varlen_workspace_bytes(w.B, w.H_q, w.H_kv, 2048)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)
    o, lse = _run(x, w, workspace=ws)
    rows = 32                               # G = 8: 8 heads x 32 positions per workgroup
    n_qblk = -(-2048 // rows)
    lst = ws[:4 * w.B * n_qblk].view(torch.int32).cpu().tolist()
    assert sorted(lst) == list(range(w.B * n_qblk))
    tiles = [_item_tiles(w, i, n_qblk, rows) for i in lst]
    assert all(a >= b for a, b in zip(tiles, tiles[1:]))
    assert tiles[0] == -(-20000 // 64)      # the 512-token chunk over 20000 keys leads
    assert tiles[-1] == 0                   # blocks past a chunk's end come last
    _check_all(x, w, o, lse, "work list batch")


def test_prefill_varlen_work_list_large_batch():
    """More sequences than the pre-pass stages in LDS (4100 > 4096): it reads
    the lengths from global memory instead; the list is still a sorted
    permutation and every chunk matches the oracle."""
    B = 4100
    g = torch.Generator().manual_seed(3800)
    lens = (torch.randint(1, 41, (B,), generator=g)).tolist()
    q_lens = [min(L, int(x)) for L, x in zip(lens, torch.randint(0, 3, (B,), generator=g))]
    w = _workload(8, 1, q_lens, lens, 40)
    banner("prefill_varlen_work_list_large_batch", B)
    x = inputs.make_prefill_varlen(w, device=DEV, seed=3800)
    need = gq.prefill_varlen_workspace_bytes(B, 8, 1, max(q_lens))
    ws = torch.full((need,), 0x55, dtype=torch.uint8, device=DEV)
    o, lse = _run(x, w, workspace=ws)
    lst = ws[:4 * B].view(torch.int32).cpu().tolist()     # one 32-position block per sequence
    assert sorted(lst) == list(range(B))
    tiles = [_item_tiles(w, i, 1, 32) for i in lst]
    assert all(a >= b for a, b in zip(tiles, tiles[1:]))
    _check_all(x, w, o, lse, "large batch")
