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

EDGE_ROWS = (0, 1, 63, 64, 127, 128, 4095, 8191)


def _run(x, w, kv=None):
    o, lse = gq.prefill(x["q"], x["k"], x["v"], S_kv=w.S_kv, causal=w.causal,
                        causal_offset=w.offset, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    return o, lse


def _pairs(w, n, seed):
    """``n`` seeded (head, row) pairs spread over all heads, plus every edge
    row on every head."""
    rows = inputs.sample_rows(w.S_q, n, seed)
    g = torch.Generator().manual_seed(seed + 1)
    heads = torch.randperm(n, generator=g).remainder(w.H_q).tolist()
    pairs = {(h, r) for h, r in zip(heads, rows)}
    for r in EDGE_ROWS:
        if r < w.S_q:
            for h in range(w.H_q):
                pairs.add((h, r))
    by_head = {}
    for h, r in sorted(pairs):
        by_head.setdefault(h, []).append(r)
    return by_head


def _check_sampled(x, w, o, lse, by_head, what):
    q32, k32, v32 = np32(x["q"]), np32(x["k"]), np32(x["v"])
    got, want, got_l, want_l = [], [], [], []
    for h, rows in by_head.items():
        rows = np.asarray(rows)
        ro, rl = oracle.prefill(q32, k32, v32, w.S_kv, w.scale, causal=w.causal,
                                causal_offset=w.offset, rows=rows, heads=[h])
        got.append(np32(o[:, h, rows]).reshape(-1, w.d))
        want.append(ro[:, 0].reshape(-1, w.d))
        got_l.append(np32(lse[:, h, rows]).reshape(-1))
        want_l.append(rl[:, 0].reshape(-1))
    check_bf16(np.concatenate(got), np.concatenate(want), what)
    check_lse(np.concatenate(got_l), np.concatenate(want_l), what, LSE_ATOL_BF16)


@pytest.mark.parametrize("name", ["prefill_causal_8k", "prefill_chunk_64k"])
def test_prefill_workload_sampled(name):
    """Full-size prefill (the bench's launch); oracle on 512 seeded (head, row)
    pairs spanning all 64 heads plus the tile-edge rows of every head."""
    w = inputs.WORKLOADS[name]
    banner(name, "gqa_attn_prefill", f"S_q={w.S_q} S_kv={w.S_kv} offset={w.offset}")
    x = inputs.make_prefill(w, device=DEV)
    o, lse = _run(x, w)
    assert torch.isfinite(o).all()
    by_head = _pairs(w, 512, inputs.SEEDS[name])
    _check_sampled(x, w, o, lse, by_head, name)


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
