"""C-ABI host checks that need no GPU: the library loads, exports every
declared symbol, and rejects bad arguments before touching any pointer."""

import ctypes
import os
import re

import pytest

from gqa_flashattention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libgqa_attn.so not built")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
F32, BF16 = 0, 1
# Fake, 256-byte aligned device addresses: validation must reject the call
# before any of them is dereferenced or handed to the runtime.
P = ctypes.c_void_p(0x100000)
P2 = ctypes.c_void_p(0x200000)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(gqa_attn_\w+)\s*\(", text, re.M)))


def test_header_and_binding_agree():
    decl = declared_functions()
    assert decl, "no declarations parsed"
    assert set(decl) == set(binding.SIGNATURES)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), f"{name} not exported"


def test_status_strings_and_version():
    L = binding.lib()
    for s in range(6):
        assert L.gqa_attn_status_string(s)
    assert L.gqa_attn_status_string(99) == b"unknown status"
    assert L.gqa_attn_version() >= 100


def test_split_tokens_rules():
    L = binding.lib()
    assert L.gqa_attn_decode_split_tokens(1, 1, 256, 0, F32) == 64
    assert L.gqa_attn_decode_split_tokens(1, 1, 256, 64, F32) == 64
    assert L.gqa_attn_decode_split_tokens(1, 1, 256, 128, F32) == -INVALID
    assert L.gqa_attn_decode_split_tokens(1, 8, 32768, 384, BF16) == 384
    assert L.gqa_attn_decode_split_tokens(1, 8, 32768, 100, BF16) == -INVALID
    # Explicit splits are capped at 2^20 keys (32-bit per-wave byte counts).
    assert L.gqa_attn_decode_split_tokens(1, 8, 1 << 21, 1 << 20, BF16) == 1 << 20
    assert L.gqa_attn_decode_split_tokens(1, 8, 1 << 21, (1 << 20) + 128, BF16) == -INVALID
    auto = L.gqa_attn_decode_split_tokens(1, 8, 32768, 0, BF16)
    assert auto == 512
    assert L.gqa_attn_decode_split_tokens(4, 8, 131072, 0, BF16) == 1280
    assert L.gqa_attn_decode_split_tokens(1, 8, 100, 0, BF16) == 128   # tiny context
    assert L.gqa_attn_decode_split_tokens(0, 8, 100, 0, BF16) == -INVALID
    assert L.gqa_attn_decode_split_tokens(1, 8, 100, 0, 7) == -INVALID


def test_workspace_bytes():
    L = binding.lib()
    n = L.gqa_attn_decode_workspace_bytes(1, 64, 8, 128, 32768, 256, BF16)
    n_split = 32768 // 256
    assert n >= 64 * n_split * (128 + 2) * 4
    assert L.gqa_attn_decode_workspace_bytes(1, 64, 8, 64, 32768, 256, BF16) == 0
    assert L.gqa_attn_decode_workspace_bytes(1, 63, 8, 128, 32768, 256, BF16) == 0


def _decode(fn="gqa_attn_decode", **kw):
    a = dict(q=P, k=P, v=P, lens=P, o=P2, lse=None, B=1, H_q=8, H_kv=1, d=128, cap=256,
             maxlen=256, scale=0.088, dtype=BF16, chunk=0, ws=P2, wsb=1 << 30, stream=None)
    a.update(kw)
    return getattr(binding.lib(), fn)(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"],
                                         a["B"], a["H_q"], a["H_kv"], a["d"], a["cap"],
                                         a["maxlen"], a["scale"], a["dtype"], a["chunk"],
                                         a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID),
    (dict(k=None), INVALID),
    (dict(lens=None), INVALID),
    (dict(o=None), INVALID),
    (dict(q=ctypes.c_void_p(0x100008)), INVALID),        # misaligned
    (dict(lse=ctypes.c_void_p(0x100002)), INVALID),
    (dict(B=0), INVALID),
    (dict(H_kv=3), INVALID),                             # H_q % H_kv != 0
    (dict(maxlen=257), INVALID),                         # > kv_cap
    (dict(dtype=5), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(chunk=100), INVALID),
    (dict(chunk=-128), INVALID),
    (dict(d=64), UNSUPPORTED),
    (dict(H_q=32, H_kv=1), UNSUPPORTED),                 # G > 16
    (dict(ws=None), WORKSPACE),
    (dict(wsb=16), WORKSPACE),
])
@pytest.mark.parametrize("fn", ["gqa_attn_decode", "gqa_attn_decode_partial",
                                "gqa_attn_decode_combine"])
def test_decode_rejects_before_launch(kw, status, fn):
    assert _decode(fn, **kw) == status


def _prefill(**kw):
    a = dict(q=P, k=P, v=P, o=P2, lse=None, B=1, H_q=8, H_kv=2, d=128, S_q=64, S_kv=128,
             cap=128, causal=1, off=0, scale=0.088, dtype=BF16, stream=None)
    a.update(kw)
    return binding.lib().gqa_attn_prefill(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                                          a["H_q"], a["H_kv"], a["d"], a["S_q"], a["S_kv"],
                                          a["cap"], a["causal"], a["off"], a["scale"],
                                          a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID),
    (dict(v=ctypes.c_void_p(0x100004)), INVALID),
    (dict(S_q=0), INVALID),
    (dict(S_kv=129), INVALID),                           # > kv_cap
    (dict(H_kv=3), INVALID),
    (dict(causal=2), INVALID),
    (dict(off=-1), INVALID),
    (dict(off=65), INVALID),                             # offset + S_q > S_kv
    (dict(scale=float("inf")), INVALID),
    (dict(dtype=F32), UNSUPPORTED),
    (dict(d=96), UNSUPPORTED),
])
def test_prefill_rejects_before_launch(kw, status):
    assert _prefill(**kw) == status


def _varlen(**kw):
    a = dict(q=P, k=P, v=P, cu=P2, lens=P2, o=P2, lse=None, B=2, H_q=8, H_kv=2, d=128,
             total=100, maxq=64, cap=128, maxkv=128, causal=1, scale=0.088, dtype=BF16,
             ws=ctypes.c_void_p(0x300000), wsb=4096, stream=None)
    a.update(kw)
    return binding.lib().gqa_attn_prefill_varlen(
        a["q"], a["k"], a["v"], a["cu"], a["lens"], a["o"], a["lse"], a["B"], a["H_q"],
        a["H_kv"], a["d"], a["total"], a["maxq"], a["cap"], a["maxkv"], a["causal"], a["scale"],
        a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), INVALID),
    (dict(lens=None), INVALID),
    (dict(lens=ctypes.c_void_p(0x200002)), INVALID),     # int32 array misaligned
    (dict(o=ctypes.c_void_p(0x200008)), INVALID),
    (dict(B=0), INVALID),
    (dict(total=-1), INVALID),
    (dict(maxq=101), INVALID),                           # > total_q
    (dict(maxq=-1), INVALID),
    (dict(maxkv=0), INVALID),
    (dict(maxkv=129), INVALID),                          # > kv_cap
    (dict(H_kv=3), INVALID),
    (dict(causal=2), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(dtype=F32), UNSUPPORTED),
    (dict(d=64), UNSUPPORTED),
    (dict(ws=None), WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x300010)), WORKSPACE),     # not 256-byte aligned
    (dict(wsb=255), WORKSPACE),
    (dict(total=0, maxq=0, ws=None), OK),                # nothing to do: no launch
    (dict(maxq=0, ws=None), OK),
])
def test_prefill_varlen_rejects_before_launch(kw, status):
    assert _varlen(**kw) == status


def _paged_prefill(**kw):
    a = dict(q=P, k=P, v=P, table=P2, cu=P2, lens=P2, o=P2, lse=None, B=2, H_q=8, H_kv=2, d=128,
             total=100, maxq=64, page=16, max_pages=8, num_pages=20, maxkv=128, causal=1,
             scale=0.088, dtype=BF16, ws=ctypes.c_void_p(0x300000), wsb=4096, stream=None)
    a.update(kw)
    return binding.lib().gqa_attn_prefill_paged(
        a["q"], a["k"], a["v"], a["table"], a["cu"], a["lens"], a["o"], a["lse"], a["B"],
        a["H_q"], a["H_kv"], a["d"], a["total"], a["maxq"], a["page"], a["max_pages"],
        a["num_pages"], a["maxkv"], a["causal"], a["scale"], a["dtype"], a["ws"], a["wsb"],
        a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(table=None), INVALID),
    (dict(table=ctypes.c_void_p(0x200002)), INVALID),
    (dict(page=24), INVALID),                            # not a power of two
    (dict(page=8), INVALID),                             # below 16
    (dict(max_pages=0), INVALID),
    (dict(num_pages=0), INVALID),
    (dict(maxkv=129), INVALID),                          # > max_pages * page
    (dict(maxkv=0), INVALID),
    (dict(cu=None), INVALID),
    (dict(maxq=101), INVALID),
    (dict(H_kv=3), INVALID),
    (dict(dtype=F32), UNSUPPORTED),
    (dict(page=16, max_pages=9000, maxkv=16 * 8193), UNSUPPORTED),   # 8193 pages of a sequence
    (dict(ws=None), WORKSPACE),
    (dict(maxq=0, ws=None), OK),
])
def test_prefill_paged_rejects_before_launch(kw, status):
    assert _paged_prefill(**kw) == status


def test_prefill_varlen_workspace_rule():
    """One int per (sequence, query block), rounded up to 256 bytes; the
    query block is 256 rows / gcd(G, 8) heads positions."""
    L = binding.lib()
    assert L.gqa_attn_prefill_varlen_workspace_bytes(8, 64, 8, 8192) == 8 * 256 * 4
    assert L.gqa_attn_prefill_varlen_workspace_bytes(2, 8, 2, 64) == 256        # G=4: 64 rows
    assert L.gqa_attn_prefill_varlen_workspace_bytes(3, 12, 2, 1000) == 256     # G=6: 128 rows
    assert L.gqa_attn_prefill_varlen_workspace_bytes(1000, 64, 8, 100) == 16128  # 16000 up
    assert L.gqa_attn_prefill_varlen_workspace_bytes(0, 64, 8, 100) == 0


def test_multi_split_and_workspace_rules():
    L = binding.lib()
    assert L.gqa_attn_decode_multi_split_tokens(1, 64, 8, 4, 32768, 0, BF16) == 1024
    assert L.gqa_attn_decode_multi_split_tokens(4, 64, 8, 4, 131072, 0, BF16) == 2048
    assert L.gqa_attn_decode_multi_split_tokens(1, 64, 8, 4, 100, 0, BF16) == 128    # tiny context
    assert L.gqa_attn_decode_multi_split_tokens(1, 64, 8, 4, 32768, 384, BF16) == 384
    assert L.gqa_attn_decode_multi_split_tokens(1, 64, 8, 4, 32768, 200, BF16) == -INVALID
    assert L.gqa_attn_decode_multi_split_tokens(1, 64, 8, 4, 1 << 21, (1 << 20) + 128,
                                                BF16) == -INVALID
    assert L.gqa_attn_decode_multi_split_tokens(1, 64, 8, 4, 32768, 0, F32) == -UNSUPPORTED
    assert L.gqa_attn_decode_multi_split_tokens(1, 64, 8, 0, 32768, 0, BF16) == -INVALID
    assert L.gqa_attn_decode_multi_split_tokens(1, 64, 8, 9, 8, 0, BF16) == -INVALID   # T_q > L
    assert L.gqa_attn_decode_multi_split_tokens(1, 63, 8, 2, 32768, 0, BF16) == -INVALID
    # G * T_q <= 16 runs on the decode split kernel and takes its split rule.
    assert (L.gqa_attn_decode_multi_split_tokens(1, 64, 8, 2, 32768, 0, BF16)
            == L.gqa_attn_decode_split_tokens(1, 8, 32768, 0, BF16) == 512)
    n = L.gqa_attn_decode_multi_workspace_bytes(1, 64, 8, 128, 4, 32768, 1024, BF16)
    assert n >= 64 * 4 * 32 * (128 + 2) * 4
    assert L.gqa_attn_decode_multi_workspace_bytes(1, 64, 8, 128, 17, 32768, 0, BF16) == 0
    assert L.gqa_attn_decode_multi_workspace_bytes(1, 64, 8, 96, 4, 32768, 0, BF16) == 0


def _decode_multi(fn="gqa_attn_decode_multi", **kw):
    a = dict(q=P, k=P, v=P, lens=P, o=P2, lse=None, B=1, H_q=8, H_kv=1, d=128, T_q=4, cap=256,
             maxlen=256, scale=0.088, dtype=BF16, chunk=0, ws=P2, wsb=1 << 30, stream=None)
    a.update(kw)
    return getattr(binding.lib(), fn)(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"],
                                         a["B"], a["H_q"], a["H_kv"], a["d"], a["T_q"],
                                         a["cap"], a["maxlen"], a["scale"], a["dtype"],
                                         a["chunk"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID),
    (dict(v=None), INVALID),
    (dict(lens=None), INVALID),
    (dict(o=ctypes.c_void_p(0x200004)), INVALID),        # misaligned
    (dict(T_q=0), INVALID),
    (dict(T_q=300, H_q=1), INVALID),                     # T_q > max_kv_len
    (dict(maxlen=257), INVALID),                         # > kv_cap
    (dict(H_kv=3), INVALID),
    (dict(scale=float("-inf")), INVALID),
    (dict(chunk=64), INVALID),
    (dict(dtype=F32), UNSUPPORTED),
    (dict(d=64), UNSUPPORTED),
    (dict(T_q=17), UNSUPPORTED),                         # G * T_q > 128
    (dict(H_q=64, H_kv=1, T_q=3), UNSUPPORTED),
    (dict(ws=None), WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x200008)), WORKSPACE),
    (dict(wsb=1024), WORKSPACE),
])
@pytest.mark.parametrize("fn", ["gqa_attn_decode_multi", "gqa_attn_decode_multi_partial",
                                "gqa_attn_decode_multi_combine"])
def test_decode_multi_rejects_before_launch(kw, status, fn):
    assert _decode_multi(fn, **kw) == status


def _merge(**kw):
    a = dict(oa=P, la=P, ob=P2, lb=P2, oo=P, lo=None, rows=100, d=128, dtype=BF16, stream=None)
    a.update(kw)
    return binding.lib().gqa_attn_merge(a["oa"], a["la"], a["ob"], a["lb"], a["oo"], a["lo"],
                                        a["rows"], a["d"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(oa=None), INVALID),
    (dict(lb=None), INVALID),
    (dict(oo=None), INVALID),
    (dict(ob=ctypes.c_void_p(0x200008)), INVALID),      # misaligned
    (dict(lo=ctypes.c_void_p(0x200002)), INVALID),
    (dict(rows=-1), INVALID),
    (dict(dtype=3), INVALID),
    (dict(d=64), UNSUPPORTED),
    (dict(rows=0), OK),                                 # nothing to do, nothing launched
])
def test_merge_rejects_before_launch(kw, status):
    assert _merge(**kw) == status


def _paged(**kw):
    a = dict(q=P, kp=P, vp=P, bt=P2, lens=P2, o=P, lse=None, B=1, H_q=8, H_kv=1, d=128, T_q=1,
             page=64, maxp=4, npages=4, maxlen=256, scale=0.088, dtype=BF16, chunk=0, ws=P2,
             wsb=1 << 30, stream=None)
    a.update(kw)
    return binding.lib().gqa_attn_decode_paged(
        a["q"], a["kp"], a["vp"], a["bt"], a["lens"], a["o"], a["lse"], a["B"], a["H_q"],
        a["H_kv"], a["d"], a["T_q"], a["page"], a["maxp"], a["npages"], a["maxlen"], a["scale"],
        a["dtype"], a["chunk"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(bt=None), INVALID),
    (dict(kp=None), INVALID),
    (dict(bt=ctypes.c_void_p(0x200002)), INVALID),       # misaligned table
    (dict(page=48), INVALID),                            # not a power of two
    (dict(page=8), INVALID),                             # below 16
    (dict(maxp=3), INVALID),                             # 3 * 64 < max_kv_len
    (dict(npages=0), INVALID),
    (dict(T_q=300, H_q=1), INVALID),                     # T_q > max_kv_len
    (dict(chunk=64), INVALID),                           # not a multiple of 128
    (dict(page=16, maxp=16, chunk=4096, maxlen=256), INVALID),   # a wave range over 64 pages
    (dict(dtype=F32), UNSUPPORTED),
    (dict(d=64), UNSUPPORTED),
    (dict(T_q=17), UNSUPPORTED),
    (dict(ws=None), WORKSPACE),
])
def test_decode_paged_rejects_before_launch(kw, status):
    assert _paged(**kw) == status


def test_paged_split_rules():
    L = binding.lib()
    # Folds of <= 16 rows take the decode rule; larger folds the multi-token
    # rule, capped at 127 pages per split.
    assert L.gqa_attn_decode_paged_split_tokens(1, 64, 8, 1, 64, 32768, 0, BF16) == 512
    assert L.gqa_attn_decode_paged_split_tokens(1, 64, 8, 4, 64, 32768, 0, BF16) == 1024
    assert L.gqa_attn_decode_paged_split_tokens(1, 64, 8, 4, 16, 131072, 0, BF16) == 1920
    assert L.gqa_attn_decode_paged_split_tokens(1, 64, 8, 4, 16, 131072, 2048, BF16) == -INVALID
    assert L.gqa_attn_decode_paged_split_tokens(1, 64, 8, 4, 24, 131072, 0, BF16) == -INVALID


def test_decode_noalloc_rejects_oversized_before_any_device_call():
    """The allocation-free decode refuses a call whose partials exceed its
    fixed scratch with GQA_ERR_SCRATCH_LIMIT, from host arithmetic alone
    (no device is touched: this runs without a GPU)."""
    L = binding.lib()
    SCRATCH_LIMIT = 5
    need = L.gqa_attn_decode_workspace_bytes(8, 64, 8, 128, 131072, 0, BF16)
    assert need > binding.DECODE_NOALLOC_SCRATCH_BYTES
    st = L.gqa_attn_decode_noalloc(P, P, P, P, P2, None, 8, 64, 8, 128, 131072, 131072,
                                   0.088, BF16, 0, None)
    assert st == SCRATCH_LIMIT
    # The workloads it is sized for fit: four 128K-key sequences.
    assert L.gqa_attn_decode_workspace_bytes(4, 64, 8, 128, 131072, 0, BF16) <= \
        binding.DECODE_NOALLOC_SCRATCH_BYTES
