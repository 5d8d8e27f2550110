"""Prefill parity on the GPU: the HIP path through the C ABI vs the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_ATOL_BF16, banner, check_bf16, check_lse, np32
from gqa_flashattention_amd import binding as gq
from gqa_flashattention_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(x, w, kv=None):
    o, lse = gq.prefill(x["q"], x["k"], x["v"], S_kv=w.S_kv, causal=w.causal,
                        causal_offset=w.offset, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    return o, lse


def _by_kv_head(w):
    return [list(range(g * w.G, (g + 1) * w.G)) for g in range(w.H_kv)]


@pytest.fixture(scope="module")
def full_size_runs():
    """One launch of each full-size prefill workload (the bench's launch);
    inputs and results moved to the host once, shared by the per-KV-head
    checks below."""
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()
            w = inputs.WORKLOADS[name]
            banner(name, "gqa_attn_prefill", f"S_q={w.S_q} S_kv={w.S_kv} offset={w.offset}")
            x = inputs.make_prefill(w, device=DEV)
            o, lse = _run(x, w)
            assert torch.isfinite(o).all()
            host = {n: np32(x[n]) for n in ("q", "k", "v")}
            cache[name] = (w, host, np32(o), np32(lse))
            del x, o, lse
            torch.cuda.empty_cache()
        return cache[name]
    return get


@pytest.mark.parametrize("kvh", range(8))
def test_prefill_causal_8k_every_element(full_size_runs, kvh):
    """prefill_causal_8k checked on every element: all 8 192 rows of the 8
    query heads of KV head ``kvh`` (O and LSE), so every workgroup of the
    launch is compared with the oracle."""
    w, x, o, lse = full_size_runs("prefill_causal_8k")
    heads = _by_kv_head(w)[kvh]
    ro, rl = oracle.prefill(x["q"], x["k"], x["v"], w.S_kv, w.scale, causal=w.causal,
                            causal_offset=w.offset, heads=heads)
    for i, h in enumerate(heads):
        check_bf16(o[0, h], ro[0, i], f"prefill_causal_8k head {h}")
    check_lse(lse[0, heads], rl[0], f"prefill_causal_8k KV head {kvh}", LSE_ATOL_BF16)


@pytest.mark.parametrize("kvh", range(8))
def test_prefill_chunk_64k_sampled_rows_all_heads(full_size_runs, kvh):
    """prefill_chunk_64k on 512 seeded query positions, each for all 64
    heads (the 8 heads of KV head ``kvh`` here): one position in every
    32-position block (so every (KV head, position block) workgroup is
    compared), the tile-edge positions and the last row."""
    w, x, o, lse = full_size_runs("prefill_chunk_64k")
    rows = np.asarray(inputs.sample_rows_per_block(w.S_q, 512, inputs.SEEDS[w.name]))
    heads = _by_kv_head(w)[kvh]
    ro, rl = oracle.prefill(x["q"], x["k"], x["v"], w.S_kv, w.scale, causal=w.causal,
                            causal_offset=w.offset, rows=rows, heads=heads)
    for i, h in enumerate(heads):
        check_bf16(o[0, h][rows], ro[0, i], f"prefill_chunk_64k head {h}")
    check_lse(lse[0, heads][:, rows], rl[0], f"prefill_chunk_64k KV head {kvh}", LSE_ATOL_BF16)


SMALL = [
    # (B, H_q, H_kv, S_q, S_kv, kv_cap, causal, offset)
    (1, 8, 1, 1, 1, 1, True, 0),
    (1, 8, 1, 64, 64, 64, True, 0),
    (1, 8, 2, 129, 129, 160, True, 0),
    (2, 4, 4, 300, 300, 300, True, 0),
    (1, 16, 2, 77, 1000, 1000, True, 923),
    (1, 8, 1, 250, 700, 768, True, 333),
    (2, 8, 1, 200, 333, 333, False, 0),
    (1, 64, 8, 384, 384, 384, True, 0),
    (1, 8, 8, 1, 5000, 5000, True, 4999),
    (1, 16, 8, 150, 150, 150, True, 0),          # G = 2
    (1, 12, 2, 100, 400, 400, True, 300),        # G = 6: 2 heads x 4 position blocks
    (1, 32, 2, 70, 70, 70, True, 0),             # G = 16: two head groups
    (1, 8, 1, 96, 2000, 2048, False, 0),         # non-causal, long keys, ragged tail
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "_".join(map(str, c)))
def test_prefill_shapes(case):
    """Every element against the oracle: ragged query and key tails, offsets,
    non-causal, GQA group sizes 1..8, NaN past S_kv."""
    B, H_q, H_kv, S_q, S_kv, cap, causal, off = case
    w = inputs.Workload("t", "prefill", B=B, H_q=H_q, H_kv=H_kv, d=128, dtype="bf16",
                        S_q=S_q, S_kv=S_kv, causal=causal, offset=off)
    banner("prefill_shapes", case)
    x = inputs.make_prefill(w, device=DEV, seed=2000 + SMALL.index(case), kv_cap=cap)
    o, lse = _run(x, w)
    ro, rl = oracle.prefill(np32(x["q"]), np32(x["k"]), np32(x["v"]), S_kv, w.scale,
                            causal=causal, causal_offset=off)
    for b in range(B):
        check_bf16(np32(o[b]), ro[b], f"{case} seq {b}")
    check_lse(np32(lse), rl, str(case), LSE_ATOL_BF16)


def test_prefill_causal_row0_is_v0_and_deterministic():
    """Causal row 0 sees only key 0: O = V[0] bitwise.  Repeats are bitwise equal."""
    w = inputs.Workload("t", "prefill", B=1, H_q=16, H_kv=2, d=128, dtype="bf16", S_q=300,
                        S_kv=300, causal=True, offset=0)
    banner("prefill_row0")
    x = inputs.make_prefill(w, device=DEV, seed=21)
    o, lse = _run(x, w)
    for h in range(16):
        assert torch.equal(o[0, h, 0], x["v"][0, h // 8, 0]), f"head {h}"
    o2, lse2 = _run(x, w)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_prefill_row_matches_decode():
    """Prefill row i equals a decode over the offset + i + 1 keys it sees
    (both checked against the oracle's decode)."""
    w = inputs.Workload("t", "prefill", B=1, H_q=64, H_kv=8, d=128, dtype="bf16", S_q=200,
                        S_kv=1200, causal=True, offset=1000)
    banner("prefill_row_vs_decode")
    x = inputs.make_prefill(w, device=DEV, seed=22)
    o, _ = _run(x, w)
    for i in (0, 57, 199):
        L = 1000 + i + 1
        qd = x["q"][:, :, i].contiguous()
        lens = torch.tensor([L], dtype=torch.int32, device=DEV)
        od = gq.decode(qd, x["k"], x["v"], lens, max_kv_len=L, scale=w.scale)
        torch.cuda.synchronize()
        ro, _ = oracle.decode(np32(qd), np32(x["k"]), np32(x["v"]), np.array([L]), w.scale)
        check_bf16(np32(o[:, :, i]), ro, f"prefill row {i}")
        check_bf16(np32(od), ro, f"decode len {L}")


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.3])
def test_prefill_scale_sign_and_zero(scale):
    """Negative scale (applied by flipping Q's sign), zero scale (uniform
    weights over the visible keys) and a large scale, causal with an offset."""
    w = inputs.Workload("t", "prefill", B=1, H_q=16, H_kv=2, d=128, dtype="bf16", S_q=90,
                        S_kv=200, causal=True, offset=110)
    banner("prefill_scale", scale)
    x = inputs.make_prefill(w, device=DEV, seed=23)
    o, lse = gq.prefill(x["q"], x["k"], x["v"], S_kv=200, causal=True, causal_offset=110,
                        scale=scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill(np32(x["q"]), np32(x["k"]), np32(x["v"]), 200, scale, causal=True,
                            causal_offset=110)
    check_bf16(np32(o[0]), ro[0], f"scale {scale}")
    check_lse(np32(lse), rl, f"scale {scale}", LSE_ATOL_BF16)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_max_jump_moves_reference(causal):
    """Keys of one later tile scaled by 40: their scores jump far above the
    running reference, so the reference must move mid-sequence (O, l and the
    pending P rescaled).  Every element against the oracle."""
    w = inputs.Workload("t", "prefill", B=1, H_q=16, H_kv=2, d=128, dtype="bf16", S_q=200,
                        S_kv=700, causal=causal, offset=500 if causal else 0)
    banner("prefill_max_jump", causal)
    x = inputs.make_prefill(w, device=DEV, seed=24)
    x["k"][:, :, 320:384] *= 40.0          # tile 5
    x["k"][:, :, 600:610] *= 25.0          # a smaller second jump inside tile 9
    o, lse = gq.prefill(x["q"], x["k"], x["v"], S_kv=w.S_kv, causal=causal,
                        causal_offset=w.offset, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill(np32(x["q"]), np32(x["k"]), np32(x["v"]), w.S_kv, w.scale,
                            causal=causal, causal_offset=w.offset)
    check_bf16(np32(o[0]), ro[0], f"max jump causal={causal}")
    check_lse(np32(lse), rl, f"max jump causal={causal}", LSE_ATOL_BF16)


def _plant_single_head_jumps(q, k, plants, q_row_dim=2):
    """Make the scores of one query head jump far above its running
    reference in one key tile, leaving the other heads of its KV head
    nearly unaffected: the query head's component ``dim`` is set to 20 and
    the keys of the tile get 30 in that component (about 53 natural-log
    units, 76 in log2, above the rest of the row).  ``plants`` lists
    (query head, KV head, first key, dim); ``q_row_dim`` is the axis of q
    that holds the query heads' rows (q is [B, H_q, S_q, d] or
    [total_q, H_q, d])."""
    for h, kvh, k0, dim in plants:
        if q_row_dim == 2:
            q[:, h, :, dim] = 20.0
        else:
            q[:, h, dim] = 20.0
        k[:, kvh, k0:k0 + 64, dim] = 30.0


# (query head, its KV head, first key of the tile, component): tiles 4 and 6
# are the first step of a group of two steps, where the fix-up used to read
# a K ring slot that another wave may already be refilling; only one wave of
# its workgroup takes the fix-up, so the waves drift apart.
EVEN_TILE_JUMPS = ((3, 0, 256, 0), (12, 1, 384, 1))


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_max_jump_even_tile_single_head(causal):
    """One query head per KV head jumps on an even tile (the first step of a
    step pair): every element against the oracle, O and LSE."""
    w = inputs.Workload("t", "prefill", B=1, H_q=16, H_kv=2, d=128, dtype="bf16", S_q=200,
                        S_kv=700, causal=causal, offset=500 if causal else 0)
    banner("prefill_max_jump_even_tile", causal)
    x = inputs.make_prefill(w, device=DEV, seed=25)
    _plant_single_head_jumps(x["q"], x["k"], EVEN_TILE_JUMPS)
    o, lse = _run(x, w)
    ro, rl = oracle.prefill(np32(x["q"]), np32(x["k"]), np32(x["v"]), w.S_kv, w.scale,
                            causal=causal, causal_offset=w.offset)
    check_bf16(np32(o[0]), ro[0], f"even-tile jump causal={causal}")
    check_lse(np32(lse), rl, f"even-tile jump causal={causal}", LSE_ATOL_BF16)
    # The waves of a workgroup drift apart here, so a cross-wave hazard
    # shows as run-to-run differences: repeat and compare bit for bit.
    for rep in range(8):
        o2, lse2 = _run(x, w)
        assert torch.equal(o, o2) and torch.equal(lse, lse2), f"repeat {rep} differs"


@pytest.mark.parametrize("page", [0, 16, 64])
def test_prefill_varlen_and_paged_max_jump_even_tile(page):
    """The same planted jumps in a varlen batch on a contiguous cache
    (page = 0) and on paged caches: every element against the oracle, and
    the paged launches bitwise equal to the contiguous one."""
    q_lens, lens = (200, 77, 130), (700, 900, 130)
    w = inputs.Workload("t", "prefill_paged" if page else "prefill_varlen", B=3, H_q=16,
                        H_kv=2, d=128, dtype="bf16", q_lens=q_lens, lens=lens, kv_cap=960,
                        causal=True, page_size=page)
    banner("prefill_varlen_max_jump_even_tile", page)
    x = inputs.make_prefill_varlen(w, device=DEV, seed=26)
    _plant_single_head_jumps(x["q"], x["k"], EVEN_TILE_JUMPS, q_row_dim=1)
    for b, L in enumerate(lens):     # padding stays NaN
        x["k"][b, :, L:] = float("nan")
    kw = dict(max_seqlen_q=max(q_lens), max_kv_len=max(lens), causal=True, scale=w.scale,
              return_lse=True)
    oc, lc = gq.prefill_varlen(x["q"], x["k"], x["v"], x["cu_seqlens_q"], x["kv_lens"], **kw)
    torch.cuda.synchronize()
    for rep in range(4):
        o2, l2 = gq.prefill_varlen(x["q"], x["k"], x["v"], x["cu_seqlens_q"], x["kv_lens"], **kw)
        torch.cuda.synchronize()
        assert torch.equal(oc, o2) and torch.equal(lc, l2), f"repeat {rep} differs"
    if page:
        kp, vp, table = inputs.scatter_pages(w, x["k"], x["v"], page, 26, 3, DEV)
        o, lse = gq.prefill_paged(x["q"], kp, vp, table, x["cu_seqlens_q"], x["kv_lens"], **kw)
        torch.cuda.synchronize()
        assert torch.equal(o, oc) and torch.equal(lse, lc)
    ro, rl = oracle.prefill_varlen(np32(x["q"]), np32(x["k"]), np32(x["v"]),
                                   np.array(x["cu_seqlens_q"].cpu()), np.array(lens), w.scale)
    check_bf16(np32(oc), ro, f"varlen even-tile jump page={page}")
    check_lse(np32(lc), rl, f"varlen even-tile jump page={page}", LSE_ATOL_BF16)
