"""Multi-token decode parity on the GPU: gqa_attn_decode_multi through the C
ABI vs the fp64 oracle (token t of a sequence of length L sees keys
0 .. L - T_q + t)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_ATOL_BF16, banner, check_bf16, check_lse, np32
from gqa_flashattention_amd import binding as gq
from gqa_flashattention_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _oracle(x, w):
    return oracle.decode_multi(np32(x["q"]), np32(x["k"]), np32(x["v"]),
                               x["kv_lens"].cpu().numpy(), w.scale)


def _run(x, w, chunk=0, scale=None):
    o, lse = gq.decode_multi(x["q"], x["k"], x["v"], x["kv_lens"], max_kv_len=max(w.lens),
                             scale=w.scale if scale is None else scale, chunk_tokens=chunk,
                             return_lse=True)
    torch.cuda.synchronize()
    return o, lse


def _check(o, lse, ref_o, ref_lse, w, what):
    for b in range(w.B):        # relative L2 per sequence
        check_bf16(np32(o[b]), ref_o[b], f"{what} seq {b}")
    check_lse(np32(lse), ref_lse, what, LSE_ATOL_BF16)


def _workload(B, H_q, H_kv, T_q, lens, cap):
    return inputs.Workload("t", "decode_multi", B=B, H_q=H_q, H_kv=H_kv, d=128, dtype="bf16",
                           lens=lens, kv_cap=cap, T_q=T_q)


@pytest.mark.parametrize("name", ["decode_multi_llama70b_32k_t2", "decode_multi_llama70b_32k_t4",
                                  "decode_multi_llama70b_32k_t16"])
def test_decode_multi_workload(name):
    """The multi-token workloads at full size, automatic split (the bench's
    launch), every output against the oracle."""
    w = inputs.WORKLOADS[name]
    banner(name, "gqa_attn_decode_multi", f"T_q={w.T_q} lens={w.lens}")
    x = inputs.make_decode_multi(w, device=DEV)
    o, lse = _run(x, w)
    ref_o, ref_lse = _oracle(x, w)
    _check(o, lse, ref_o, ref_lse, w, name)


SMALL = [
    # (B, H_q, H_kv, T_q, lens, kv_cap, chunk)
    (1, 8, 1, 1, (1,), 1, 0),                 # one key, T_q = 1
    (1, 8, 1, 2, (2,), 40, 0),                # L = T_q: token 0 sees key 0 only
    (1, 8, 1, 4, (5,), 40, 0),                # 32 rows, one row group
    (2, 8, 2, 3, (31, 33), 64, 128),          # 24 rows
    (1, 8, 1, 5, (129,), 129, 128),           # 40 rows; split 1 holds one key, hidden from 4 tokens
    (3, 16, 2, 6, (127, 128, 1000), 1000, 256),
    (2, 8, 1, 12, (300, 17), 300, 128),       # 96 rows: four row groups, the last one padding
    (1, 64, 8, 16, (4097,), 4100, 0),         # 128 rows, automatic split
    (1, 64, 8, 8, (1000,), 1000, 256),        # 64 rows
    (2, 4, 2, 16, (40, 16), 64, 128),         # G = 2; second sequence L = T_q
    (1, 128, 1, 1, (700,), 700, 256),         # G = 128 at T_q = 1
    (1, 8, 1, 16, (2049,), 2049, 0),
]


SMALL_DECODE_KERNEL = [
    # G * T_q <= 16: these run on the decode split kernel with a per-row tail.
    (1, 8, 1, 2, (2,), 8, 0),                 # L = T_q
    (1, 8, 1, 2, (3,), 8, 0),
    (2, 8, 1, 2, (129, 257), 300, 128),       # last split holds one key: token 0 sees none of it
    (1, 8, 1, 2, (641,), 700, 512),           # wave quarter 1 of the last split: one key
    (2, 16, 4, 4, (33, 1000), 1024, 0),       # G = 4, T_q = 4
    (1, 16, 8, 8, (4097,), 4100, 0),          # G = 2, T_q = 8
    (1, 8, 8, 16, (300,), 300, 128),          # G = 1, T_q = 16
    (1, 64, 8, 2, (5000,), 5000, 0),          # Llama geometry, T_q = 2
]


@pytest.mark.parametrize("case", SMALL + SMALL_DECODE_KERNEL,
                         ids=lambda c: f"B{c[0]}_Hq{c[1]}_Hkv{c[2]}_T{c[3]}_L{c[4]}_c{c[6]}")
def test_decode_multi_shapes(case):
    """Row groups of 1, 2 and 4 (with padding rows), ragged tails, splits
    with keys hidden from some tokens, NaN-padded caches."""
    B, H_q, H_kv, T_q, lens, cap, chunk = case
    w = _workload(B, H_q, H_kv, T_q, lens, cap)
    banner("decode_multi_shapes", case)
    x = inputs.make_decode_multi(w, device=DEV, seed=2000 + (SMALL + SMALL_DECODE_KERNEL).index(case))
    o, lse = _run(x, w, chunk)
    ref_o, ref_lse = _oracle(x, w)
    _check(o, lse, ref_o, ref_lse, w, f"shapes {case}")


def test_decode_multi_t1_matches_decode():
    """T_q = 1 through gqa_attn_decode_multi against the oracle's plain
    decode, and within bf16 output rounding of gqa_attn_decode."""
    w = _workload(2, 64, 8, 1, (3000, 1234), 3000)
    banner("decode_multi_t1")
    x = inputs.make_decode_multi(w, device=DEV, seed=21)
    o, lse = _run(x, w)
    ref_o, ref_lse = oracle.decode(np32(x["q"][:, :, 0]), np32(x["k"]), np32(x["v"]),
                                   x["kv_lens"].cpu().numpy(), w.scale)
    _check(o[:, :, 0], lse[:, :, 0], ref_o, ref_lse, w, "T_q=1 vs oracle decode")
    od, ld = gq.decode(x["q"][:, :, 0].contiguous(), x["k"], x["v"], x["kv_lens"],
                       max_kv_len=3000, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    diff = (o[:, :, 0].float() - od.float()).abs().max().item()
    assert diff <= 2 * 2.0 ** -8 * od.float().abs().max().item() + 1e-6, diff
    assert (lse[:, :, 0] - ld).abs().max().item() <= LSE_ATOL_BF16


BELOW_BOUND = [
    # (T_q, L, max_kv_len, chunk): one sequence shorter than the host bound,
    # NaN-padded past L up to the capacity (4096)
    (4, 1000, 4000, 128),     # the split holding L: its second step reaches past L
    (4, 930, 4000, 128),      # ... its first step reaches past L, and is its only one
    (4, 33, 4000, 0),         # one split holds the whole sequence; all others are empty
    (4, 4000, 4000, 0),       # L equal to the bound
    (3, 517, 3333, 256),      # 24 rows
    (8, 700, 4000, 256),      # two row groups
    (16, 2049, 4000, 0),      # four row groups
]


@pytest.mark.parametrize("case", BELOW_BOUND, ids=lambda c: f"T{c[0]}_L{c[1]}_max{c[2]}_c{c[3]}")
def test_decode_multi_single_sequence_below_host_bound(case):
    """A single sequence whose device length is below the host bound
    max_kv_len: the grid covers the bound, so some splits hold keys past L
    or none at all; every key past L must get weight zero (the NaN padding
    there must not reach the output) and the empty splits must not count."""
    T_q, L, max_len, chunk = case
    w = _workload(1, 64, 8, T_q, (L,), 4096)
    banner("decode_multi_below_bound", case)
    x = inputs.make_decode_multi(w, device=DEV, seed=3000 + BELOW_BOUND.index(case))
    o, lse = gq.decode_multi(x["q"], x["k"], x["v"], x["kv_lens"], max_kv_len=max_len,
                             scale=w.scale, chunk_tokens=chunk, return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_lse = _oracle(x, w)
    _check(o, lse, ref_o, ref_lse, w, f"below bound {case}")


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.35])
def test_decode_multi_scales(scale):
    """Negative (applied by flipping Q's sign), zero (uniform weights) and
    large scales against the oracle."""
    w = _workload(1, 32, 4, 6, (777,), 800)
    banner("decode_multi_scale", scale)
    x = inputs.make_decode_multi(w, device=DEV, seed=22)
    o, lse = _run(x, w, scale=scale)
    ref_o, ref_lse = oracle.decode_multi(np32(x["q"]), np32(x["k"]), np32(x["v"]),
                                         x["kv_lens"].cpu().numpy(), scale)
    _check(o, lse, ref_o, ref_lse, w, f"scale {scale}")


@pytest.mark.parametrize("chunk,T_q", [(0, 8), (128, 8), (0, 2), (128, 2)])
def test_decode_multi_max_jump(chunk, T_q):
    """Keys of a later stretch scaled by 40 (and a few by 25, some inside the
    causal tail): the running max (T_q = 2, decode kernel) or the per-row
    reference (T_q = 8, 64 rows) moves inside and between splits."""
    w = _workload(2, 16, 2, T_q, (5000, 3100), 5000)
    banner("decode_multi_max_jump", chunk, T_q)
    x = inputs.make_decode_multi(w, device=DEV, seed=23)
    x["k"][:, :, 3000:3100] *= 40.0
    x["k"][:, :, 4500:4510] *= 25.0
    x["k"][0, :, 4995:4998] *= 30.0       # visible to the later tokens only
    o, lse = _run(x, w, chunk)
    ref_o, ref_lse = _oracle(x, w)
    _check(o, lse, ref_o, ref_lse, w, f"max jump chunk={chunk}")


def test_decode_multi_split_invariance_and_determinism():
    """Any split size reaches the oracle; the same split is bitwise repeatable.  128-key
    splits of 9000 keys give 71 partials per row: the combine's second load round."""
    w = _workload(2, 64, 8, 4, (9000, 3001), 9000)
    banner("decode_multi_split_invariance")
    x = inputs.make_decode_multi(w, device=DEV, seed=24)
    ref_o, ref_lse = _oracle(x, w)
    for chunk in (128, 384, 1024, 0):
        o, lse = _run(x, w, chunk)
        _check(o, lse, ref_o, ref_lse, w, f"chunk {chunk}")
        o2, lse2 = _run(x, w, chunk)
        assert torch.equal(o, o2) and torch.equal(lse, lse2), f"chunk {chunk} not deterministic"


@pytest.mark.parametrize("T_q", [2, 4])
def test_decode_multi_tokens_are_causal(T_q):
    """Changing the last cache row (the newest token's K/V) changes only the
    newest token's outputs: earlier tokens never see it (decode kernel at
    T_q = 2, multi-token kernel at T_q = 4)."""
    w = _workload(1, 64, 8, T_q, (1500,), 1500)
    banner("decode_multi_causal_tail", T_q)
    x = inputs.make_decode_multi(w, device=DEV, seed=25)
    o1, _ = _run(x, w)
    x["k"][:, :, 1499] = torch.randn_like(x["k"][:, :, 1499]) * 3
    x["v"][:, :, 1499] = torch.randn_like(x["v"][:, :, 1499]) * 3
    o2, _ = _run(x, w)
    assert torch.equal(o1[:, :, :T_q - 1], o2[:, :, :T_q - 1])
    assert not torch.equal(o1[:, :, T_q - 1], o2[:, :, T_q - 1])


def test_decode_multi_phases_equal_one_call():
    """gqa_attn_decode_multi_partial then _combine on one stream, with a
    workspace filled with garbage first, is gqa_attn_decode_multi."""
    w = _workload(3, 64, 8, 8, (4000, 70, 2500), 4096)
    banner("decode_multi_phases")
    x = inputs.make_decode_multi(w, device=DEV, seed=26)
    need = gq.decode_multi_workspace_bytes(3, 64, 8, 128, 8, 4000, 0, gq.DTYPE_BF16)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    kw = dict(max_kv_len=4000, scale=w.scale, return_lse=True, workspace=ws)
    one, l1 = gq.decode_multi(x["q"], x["k"], x["v"], x["kv_lens"], **kw)
    two = torch.empty_like(one)
    l2 = torch.empty_like(l1)
    gq.decode_multi(x["q"], x["k"], x["v"], x["kv_lens"], out=two, lse=l2, phase="partial", **kw)
    gq.decode_multi(x["q"], x["k"], x["v"], x["kv_lens"], out=two, lse=l2, phase="combine", **kw)
    torch.cuda.synchronize()
    assert torch.equal(one, two) and torch.equal(l1, l2)
    ref_o, ref_lse = _oracle(x, w)
    _check(one, l1, ref_o, ref_lse, w, "phases")
