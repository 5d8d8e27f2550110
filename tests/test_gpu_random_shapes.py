"""Seeded random shapes on every compute entry point, each against the fp64
oracle on every element: group sizes, batch sizes, cache lengths, causal
offsets, split sizes and chunk mixes drawn from one fixed generator, so the
case list is the same on every run and each case is named by its shape.

The hand-picked cases of the other GPU tests aim at known edges (one key, a
split holding one key, tile boundaries); these draw the shapes between
them, at sizes the oracle finishes in well under a second."""

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

_rng = np.random.RandomState(20261202)


def _pick(seq):
    return seq[_rng.randint(len(seq))]


def _heads(max_g=16, max_hq=64):
    H_kv = int(_pick([1, 2, 4, 8]))
    gs = [g for g in (1, 2, 3, 4, 5, 6, 7, 8, 12, 16) if g <= max_g and g * H_kv <= max_hq]
    G = int(_pick(gs))
    return G * H_kv, H_kv


def _decode_cases(n, dtype, max_len, chunks):
    out = []
    for _ in range(n):
        H_q, H_kv = _heads()
        B = int(_rng.randint(1, 4))
        lens = tuple(int(x) for x in _rng.randint(1, max_len + 1, size=B))
        cap = max(lens) + int(_rng.randint(0, 200))
        out.append((B, H_q, H_kv, lens, cap, dtype, int(_pick(chunks))))
    return out


def _multi_cases(n):
    out = []
    for _ in range(n):
        T_q = int(_rng.randint(2, 17))
        H_kv = int(_pick([1, 2, 4, 8]))
        gs = [g for g in (1, 2, 4, 8) if g * T_q <= 128 and g * H_kv <= 64]
        G = int(_pick(gs))
        B = int(_rng.randint(1, 3))
        lens = tuple(int(x) for x in _rng.randint(T_q, 3000, size=B))
        cap = max(lens) + int(_rng.randint(0, 100))
        out.append((B, G * H_kv, H_kv, T_q, lens, cap, int(_pick([0, 128, 256, 512, 1024]))))
    return out


def _prefill_cases(n):
    out = []
    for _ in range(n):
        H_kv = int(_pick([1, 2, 4]))
        G = int(_pick([1, 2, 3, 4, 6, 8, 16]))
        B = int(_rng.randint(1, 3))
        S_q = int(_rng.randint(1, 700))
        causal = bool(_rng.randint(2))
        if causal:
            off = int(_rng.randint(0, 1300))
            S_kv = off + S_q + int(_rng.randint(0, 100))
        else:
            off = 0
            S_kv = int(_rng.randint(1, 2000))
        cap = S_kv + int(_rng.randint(0, 64))
        out.append((B, G * H_kv, H_kv, S_q, S_kv, cap, causal, off))
    return out


def _varlen_cases(n):
    out = []
    for _ in range(n):
        H_kv = int(_pick([1, 2, 8]))
        G = int(_pick([1, 2, 4, 8]))
        B = int(_rng.randint(1, 6))
        q_lens = tuple(int(x) for x in _rng.randint(0, 300, size=B))
        lens = tuple(q + int(_rng.randint(0, 1500)) for q in q_lens)
        if max(q_lens) == 0:
            q_lens = (1,) + q_lens[1:]
            lens = (max(lens[0], 1),) + lens[1:]
        cap = max(lens) + int(_rng.randint(0, 64))
        out.append((G * H_kv, H_kv, q_lens, lens, cap, bool(_rng.randint(2))))
    return out


def _paged_decode_cases(n):
    out = []
    for _ in range(n):
        T_q = int(_pick([1, 1, 2, 4, 8, 16]))
        H_kv = int(_pick([1, 2, 4, 8]))
        gs = [g for g in (1, 2, 4, 8) if g * T_q <= 128 and g * H_kv <= 64]
        G = int(_pick(gs))
        B = int(_rng.randint(1, 4))
        lens = tuple(int(x) for x in _rng.randint(T_q, 3000, size=B))
        cap = max(lens) + int(_rng.randint(0, 100))
        out.append((B, G * H_kv, H_kv, T_q, lens, cap, int(_pick([16, 32, 64, 128, 256]))))
    return out


DECODE_BF16 = _decode_cases(10, "bf16", 4000, [0, 128, 256, 384, 512, 768, 1024])
DECODE_F32 = _decode_cases(4, "f32", 2000, [0, 64])
MULTI = _multi_cases(8)
PREFILL = _prefill_cases(8)
VARLEN = _varlen_cases(4)
PAGED_DECODE = _paged_decode_cases(6)
PAGED_PREFILL = [c + (int(_pick([16, 32, 64, 128])),) for c in _varlen_cases(3)]


def _id(c):
    return "_".join("-".join(map(str, x)) if isinstance(x, tuple) else str(x) for x in c)


@pytest.mark.parametrize("case", DECODE_BF16 + DECODE_F32, ids=_id)
def test_random_decode(case):
    B, H_q, H_kv, lens, cap, dt, chunk = case
    w = inputs.Workload("t", "decode", B=B, H_q=H_q, H_kv=H_kv, d=128, dtype=dt, lens=lens,
                        kv_cap=cap)
    banner("random_decode", case)
    x = inputs.make_decode(w, device=DEV, seed=7000 + (DECODE_BF16 + DECODE_F32).index(case))
    o, lse = gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], max_kv_len=max(lens), scale=w.scale,
                       chunk_tokens=chunk, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(np32(x["q"]), np32(x["k"]), np32(x["v"]), np.array(lens), w.scale)
    if dt == "f32":
        check_f32(np32(o), ro, str(case))
        check_lse(np32(lse), rl, str(case), LSE_ATOL_F32)
    else:
        for b in range(B):
            check_bf16(np32(o[b]), ro[b], f"{case} seq {b}")
        check_lse(np32(lse), rl, str(case), LSE_ATOL_BF16)


@pytest.mark.parametrize("case", MULTI, ids=_id)
def test_random_decode_multi(case):
    B, H_q, H_kv, T_q, lens, cap, chunk = case
    w = inputs.Workload("t", "decode_multi", B=B, H_q=H_q, H_kv=H_kv, d=128, dtype="bf16",
                        lens=lens, kv_cap=cap, T_q=T_q)
    banner("random_decode_multi", case)
    x = inputs.make_decode_multi(w, device=DEV, seed=7100 + MULTI.index(case))
    o, lse = gq.decode_multi(x["q"], x["k"], x["v"], x["kv_lens"], max_kv_len=max(lens),
                             scale=w.scale, chunk_tokens=chunk, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_multi(np32(x["q"]), np32(x["k"]), np32(x["v"]), np.array(lens),
                                 w.scale)
    for b in range(B):
        check_bf16(np32(o[b]), ro[b], f"{case} seq {b}")
    check_lse(np32(lse), rl, str(case), LSE_ATOL_BF16)


@pytest.mark.parametrize("case", PREFILL, ids=_id)
def test_random_prefill(case):
    B, H_q, H_kv, S_q, S_kv, cap, causal, off = case
    w = inputs.Workload("t", "prefill", B=B, H_q=H_q, H_kv=H_kv, d=128, dtype="bf16", S_q=S_q,
                        S_kv=S_kv, causal=causal, offset=off)
    banner("random_prefill", case)
    x = inputs.make_prefill(w, device=DEV, seed=7200 + PREFILL.index(case), kv_cap=cap)
    o, lse = gq.prefill(x["q"], x["k"], x["v"], S_kv=S_kv, causal=causal, causal_offset=off,
                        scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill(np32(x["q"]), np32(x["k"]), np32(x["v"]), S_kv, w.scale,
                            causal=causal, causal_offset=off)
    for b in range(B):
        check_bf16(np32(o[b]), ro[b], f"{case} seq {b}")
    check_lse(np32(lse), rl, str(case), LSE_ATOL_BF16)


@pytest.mark.parametrize("case", VARLEN, ids=_id)
def test_random_prefill_varlen(case):
    H_q, H_kv, q_lens, lens, cap, causal = case
    w = inputs.Workload("t", "prefill_varlen", B=len(q_lens), H_q=H_q, H_kv=H_kv, d=128,
                        dtype="bf16", q_lens=q_lens, lens=lens, kv_cap=cap, causal=causal)
    banner("random_prefill_varlen", case)
    x = inputs.make_prefill_varlen(w, device=DEV, seed=7300 + VARLEN.index(case))
    o, lse = gq.prefill_varlen(x["q"], x["k"], x["v"], x["cu_seqlens_q"], x["kv_lens"],
                               max_seqlen_q=max(max(q_lens), 1), max_kv_len=max(max(lens), 1),
                               causal=causal, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_varlen(np32(x["q"]), np32(x["k"]), np32(x["v"]),
                                   x["cu_seqlens_q"].cpu().numpy(), np.array(lens), w.scale,
                                   causal=causal)
    cu = x["cu_seqlens_q"].cpu().tolist()
    for b in range(len(q_lens)):
        if cu[b + 1] == cu[b]:
            continue
        check_bf16(np32(o[cu[b]:cu[b + 1]]), ro[cu[b]:cu[b + 1]], f"{case} seq {b}")
        check_lse(np32(lse[cu[b]:cu[b + 1]]), rl[cu[b]:cu[b + 1]], f"{case} seq {b}",
                  LSE_ATOL_BF16)


@pytest.mark.parametrize("case", PAGED_DECODE, ids=_id)
def test_random_decode_paged(case):
    B, H_q, H_kv, T_q, lens, cap, page = case
    w = inputs.Workload("t", "decode_multi", B=B, H_q=H_q, H_kv=H_kv, d=128, dtype="bf16",
                        lens=lens, kv_cap=cap, T_q=T_q)
    banner("random_decode_paged", case)
    x = inputs.make_decode_paged(w, page, device=DEV, seed=7400 + PAGED_DECODE.index(case))
    o, lse = gq.decode_paged(x["q"], x["k_pages"], x["v_pages"], x["block_table"], x["kv_lens"],
                             max_kv_len=max(lens), scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(np32(x["q"]), np32(x["k_pages"]), np32(x["v_pages"]),
                                 x["block_table"].cpu().numpy(), np.array(lens), page, w.scale)
    for b in range(B):
        check_bf16(np32(o[b]), ro[b], f"{case} seq {b}")
    check_lse(np32(lse), rl, str(case), LSE_ATOL_BF16)


@pytest.mark.parametrize("case", PAGED_PREFILL, ids=_id)
def test_random_prefill_paged(case):
    H_q, H_kv, q_lens, lens, cap, causal, page = case
    w = inputs.Workload("t", "prefill_paged", B=len(q_lens), H_q=H_q, H_kv=H_kv, d=128,
                        dtype="bf16", q_lens=q_lens, lens=lens, kv_cap=cap, causal=causal,
                        page_size=page)
    banner("random_prefill_paged", case)
    x = inputs.make_prefill_paged(w, page, device=DEV, seed=7500 + PAGED_PREFILL.index(case))
    o, lse = gq.prefill_paged(x["q"], x["k_pages"], x["v_pages"], x["block_table"],
                              x["cu_seqlens_q"], x["kv_lens"], max_seqlen_q=max(max(q_lens), 1),
                              max_kv_len=max(max(lens), 1), causal=causal, scale=w.scale,
                              return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_paged(np32(x["q"]), np32(x["k_pages"]), np32(x["v_pages"]),
                                  x["block_table"].cpu().numpy(), x["cu_seqlens_q"].cpu().numpy(),
                                  np.array(lens), page, w.scale, causal=causal)
    cu = x["cu_seqlens_q"].cpu().tolist()
    for b in range(len(q_lens)):
        if cu[b + 1] == cu[b]:
            continue
        check_bf16(np32(o[cu[b]:cu[b + 1]]), ro[cu[b]:cu[b + 1]], f"{case} seq {b}")
        check_lse(np32(lse[cu[b]:cu[b + 1]]), rl[cu[b]:cu[b + 1]], f"{case} seq {b}",
                  LSE_ATOL_BF16)
