"""Thin ctypes binding over ``libgqa_attn.so``.

Argument marshalling only: torch tensors supply device pointers, shapes and
the current HIP stream; every step of the computation runs in the library's
HIP kernels.  There is no CPU or PyTorch fallback: if the library is missing
or a call fails, an exception says so.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgqa_attn.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1

STATUS_NAMES = {0: "GQA_OK", 1: "GQA_ERR_INVALID_ARG", 2: "GQA_ERR_UNSUPPORTED",
                3: "GQA_ERR_WORKSPACE", 4: "GQA_ERR_HIP", 5: "GQA_ERR_SCRATCH_LIMIT"}

# Size of the fixed device scratch of gqa_attn_decode_noalloc
# (GQA_DECODE_NOALLOC_SCRATCH_BYTES in the header).
DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20

# Every symbol include/gqa_attn.h declares, with its ctypes signature.
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "gqa_attn_status_string": (ctypes.c_char_p, [_i]),
    "gqa_attn_version": (_i, []),
    "gqa_attn_decode_split_tokens": (_i, [_i, _i, _i, _i, _i]),
    "gqa_attn_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "gqa_attn_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i,
                             _i, _vp, _sz, _vp]),
    "gqa_attn_decode_fused": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i,
                                   _i, _vp, _sz, _vp]),
    "gqa_attn_decode_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                                     _i, _i, _vp]),
    "gqa_attn_decode_partial": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                                     _i, _i, _vp, _sz, _vp]),
    "gqa_attn_decode_combine": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                                     _i, _i, _vp, _sz, _vp]),
    "gqa_attn_prefill": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                              _f, _i, _vp]),
    "gqa_attn_prefill_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                     _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "gqa_attn_prefill_varlen_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "gqa_attn_prefill_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                    _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "gqa_attn_merge": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_longlong, _i, _i, _vp]),
    "gqa_attn_decode_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                                   _i, _i, _f, _i, _i, _vp, _sz, _vp]),
    "gqa_attn_decode_paged_partial": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                           _i, _i, _i, _i, _f, _i, _i, _vp, _sz, _vp]),
    "gqa_attn_decode_paged_combine": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                           _i, _i, _i, _i, _f, _i, _i, _vp, _sz, _vp]),
    "gqa_attn_decode_paged_split_tokens": (_i, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "gqa_attn_decode_paged_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "gqa_attn_decode_multi_split_tokens": (_i, [_i, _i, _i, _i, _i, _i, _i]),
    "gqa_attn_decode_multi_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "gqa_attn_decode_multi": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f,
                                   _i, _i, _vp, _sz, _vp]),
    "gqa_attn_decode_multi_partial": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                           _i, _f, _i, _i, _vp, _sz, _vp]),
    "gqa_attn_decode_multi_combine": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                           _i, _f, _i, _i, _vp, _sz, _vp]),
}


class GQAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} "
                         f"({lib().gqa_attn_status_string(status).decode()})")


_LIB = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m gqa_flashattention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise GQAError(status, where)


def _require_gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("gqa_flashattention_amd runs on the GPU only: got a CPU tensor")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _expect(t, name, shape, dtype, device):
    """Check one tensor argument on the host before any pointer reaches the
    library: a wrong shape, dtype, device or stride would otherwise become an
    out-of-bounds device access instead of an error."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _expect_workspace(ws, device, need):
    """A caller-supplied workspace: contiguous, on the device, at least
    ``need`` bytes (the library checks the size too)."""
    _expect(ws, "workspace", None, None, device)
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, "
                         f"{need} needed")


def _check_kv(q, k, v, batch):
    """K and V: 4-D, the same shape, q's dtype and device, ``d`` of q and
    batch ``batch`` (None: not checked, e.g. a page pool)."""
    if k.dim() != 4:
        raise ValueError(f"k must be 4-D, got shape {tuple(k.shape)}")
    _expect(k, "k", None, q.dtype, q.device)
    _expect(v, "v", k.shape, q.dtype, q.device)
    if k.shape[3] != q.shape[-1]:
        raise ValueError(f"k/v head dimension {k.shape[3]} differs from q's {q.shape[-1]}")
    if batch is not None and k.shape[0] != batch:
        raise ValueError(f"k/v hold {k.shape[0]} sequences, q has {batch}")


def decode_split_tokens(B, H_kv, max_kv_len, chunk_tokens=0, dtype=DTYPE_BF16) -> int:
    r = lib().gqa_attn_decode_split_tokens(B, H_kv, max_kv_len, chunk_tokens, dtype)
    if r < 0:
        raise GQAError(-r, "gqa_attn_decode_split_tokens")
    return r


def decode_workspace_bytes(B, H_q, H_kv, d, max_kv_len, chunk_tokens=0, dtype=DTYPE_BF16) -> int:
    n = lib().gqa_attn_decode_workspace_bytes(B, H_q, H_kv, d, max_kv_len, chunk_tokens, dtype)
    if n == 0:
        raise GQAError(1, "gqa_attn_decode_workspace_bytes")
    return n


def decode(q, k_cache, v_cache, kv_lens, max_kv_len=None, scale=None, chunk_tokens=0,
           return_lse=False, out=None, lse=None, workspace=None, stream=None, phase="both"):
    """``gqa_attn_decode`` on torch tensors.

    q ``[B,H_q,d]``, k_cache/v_cache ``[B,H_kv,kv_cap,d]`` (same dtype, bf16 or
    fp32), kv_lens ``[B]`` int32 on the device.  ``max_kv_len`` defaults to
    ``kv_cap``.  ``phase`` = "partial" or "combine" issues only that launch
    (``gqa_attn_decode_partial`` / ``_combine``; pass the same ``workspace``
    to both); "fused" runs ``gqa_attn_decode_fused`` (one launch; a
    caller-supplied workspace must have been zero-filled before its first
    fused call).  Returns ``o`` (and ``lse`` when ``return_lse``).
    """
    _require_gpu(q)
    if q.dim() != 3:
        raise ValueError(f"q must be [B, H_q, d], got shape {tuple(q.shape)}")
    B, H_q, d = q.shape
    dt = _dtype_code(q)
    _check_kv(q, k_cache, v_cache, B)
    _, H_kv, kv_cap, _ = k_cache.shape
    _expect(kv_lens, "kv_lens", (B,), torch.int32, q.device)
    max_kv_len = kv_cap if max_kv_len is None else int(max_kv_len)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, "out", q.shape, q.dtype, q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=q.device)
    if return_lse:
        _expect(lse, "lse", (B, H_q), torch.float32, q.device)
    need = decode_workspace_bytes(B, H_q, H_kv, d, max_kv_len, chunk_tokens, dt)
    if workspace is None:
        # zeros: the fused form's arrival counters must start at zero (every
        # fused call leaves them zero); the other phases ignore them.
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    _expect_workspace(workspace, q.device, need)
    fn = {"both": "gqa_attn_decode", "partial": "gqa_attn_decode_partial",
          "combine": "gqa_attn_decode_combine", "fused": "gqa_attn_decode_fused"}[phase]
    st = getattr(lib(), fn)(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_lens), _ptr(out),
                            _ptr(lse) if return_lse else None, B, H_q, H_kv, d, kv_cap,
                            max_kv_len, scale, dt, chunk_tokens, _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, fn)
    return (out, lse) if return_lse else out


def decode_noalloc(q, k_cache, v_cache, kv_lens, out, max_kv_len=None, scale=None,
                   chunk_tokens=0, lse=None, stream=None):
    """``gqa_attn_decode_noalloc`` on torch tensors: :func:`decode` without a
    workspace (the library's fixed per-device scratch holds the partials)
    and without allocating anything here either -- ``out`` (and ``lse``,
    when the LSE is wanted) are the caller's.  Calls that overlap in time on
    one device race on the shared scratch.  Returns ``out`` (and ``lse``
    when given)."""
    _require_gpu(q)
    if q.dim() != 3:
        raise ValueError(f"q must be [B, H_q, d], got shape {tuple(q.shape)}")
    B, H_q, d = q.shape
    dt = _dtype_code(q)
    _check_kv(q, k_cache, v_cache, B)
    _, H_kv, kv_cap, _ = k_cache.shape
    _expect(kv_lens, "kv_lens", (B,), torch.int32, q.device)
    _expect(out, "out", q.shape, q.dtype, q.device)
    if lse is not None:
        _expect(lse, "lse", (B, H_q), torch.float32, q.device)
    max_kv_len = kv_cap if max_kv_len is None else int(max_kv_len)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib().gqa_attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_lens),
                                       _ptr(out), _ptr(lse), B, H_q, H_kv, d, kv_cap, max_kv_len,
                                       scale, dt, chunk_tokens, _stream(stream))
    _check(st, "gqa_attn_decode_noalloc")
    return (out, lse) if lse is not None else out


def decode_multi_split_tokens(B, H_q, H_kv, T_q, max_kv_len, chunk_tokens=0,
                              dtype=DTYPE_BF16) -> int:
    r = lib().gqa_attn_decode_multi_split_tokens(B, H_q, H_kv, T_q, max_kv_len, chunk_tokens,
                                                 dtype)
    if r < 0:
        raise GQAError(-r, "gqa_attn_decode_multi_split_tokens")
    return r


def decode_multi_workspace_bytes(B, H_q, H_kv, d, T_q, max_kv_len, chunk_tokens=0,
                                 dtype=DTYPE_BF16) -> int:
    n = lib().gqa_attn_decode_multi_workspace_bytes(B, H_q, H_kv, d, T_q, max_kv_len,
                                                    chunk_tokens, dtype)
    if n == 0:
        raise GQAError(1, "gqa_attn_decode_multi_workspace_bytes")
    return n


def decode_multi(q, k_cache, v_cache, kv_lens, max_kv_len=None, scale=None, chunk_tokens=0,
                 return_lse=False, out=None, lse=None, workspace=None, stream=None,
                 phase="both"):
    """``gqa_attn_decode_multi`` on torch tensors.

    q ``[B,H_q,T_q,d]`` bf16 (token t of a sequence of length L sits at
    position L - T_q + t), k_cache/v_cache ``[B,H_kv,kv_cap,d]`` bf16 holding
    the new tokens' rows, kv_lens ``[B]`` int32 on the device.  ``phase`` as
    for :func:`decode`.  Returns ``o`` (and ``lse`` ``[B,H_q,T_q]`` when
    ``return_lse``).
    """
    _require_gpu(q)
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H_q, T_q, d], got shape {tuple(q.shape)}")
    B, H_q, T_q, d = q.shape
    dt = _dtype_code(q)
    _check_kv(q, k_cache, v_cache, B)
    _, H_kv, kv_cap, _ = k_cache.shape
    _expect(kv_lens, "kv_lens", (B,), torch.int32, q.device)
    max_kv_len = kv_cap if max_kv_len is None else int(max_kv_len)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, "out", q.shape, q.dtype, q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, H_q, T_q), dtype=torch.float32, device=q.device)
    if return_lse:
        _expect(lse, "lse", (B, H_q, T_q), torch.float32, q.device)
    need = decode_multi_workspace_bytes(B, H_q, H_kv, d, T_q, max_kv_len, chunk_tokens, dt)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _expect_workspace(workspace, q.device, need)
    fn = {"both": "gqa_attn_decode_multi", "partial": "gqa_attn_decode_multi_partial",
          "combine": "gqa_attn_decode_multi_combine"}[phase]
    st = getattr(lib(), fn)(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_lens), _ptr(out),
                            _ptr(lse) if return_lse else None, B, H_q, H_kv, d, T_q, kv_cap,
                            max_kv_len, scale, dt, chunk_tokens, _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, fn)
    return (out, lse) if return_lse else out


def decode_paged_split_tokens(B, H_q, H_kv, T_q, page_size, max_kv_len, chunk_tokens=0,
                              dtype=DTYPE_BF16) -> int:
    r = lib().gqa_attn_decode_paged_split_tokens(B, H_q, H_kv, T_q, page_size, max_kv_len,
                                                 chunk_tokens, dtype)
    if r < 0:
        raise GQAError(-r, "gqa_attn_decode_paged_split_tokens")
    return r


def decode_paged_workspace_bytes(B, H_q, H_kv, d, T_q, page_size, max_kv_len, chunk_tokens=0,
                                 dtype=DTYPE_BF16) -> int:
    n = lib().gqa_attn_decode_paged_workspace_bytes(B, H_q, H_kv, d, T_q, page_size, max_kv_len,
                                                    chunk_tokens, dtype)
    if n == 0:
        raise GQAError(1, "gqa_attn_decode_paged_workspace_bytes")
    return n


def decode_paged(q, k_pages, v_pages, block_table, kv_lens, max_kv_len, scale=None,
                 chunk_tokens=0, return_lse=False, out=None, lse=None, workspace=None,
                 stream=None, phase="both"):
    """``gqa_attn_decode_paged`` on torch tensors.

    q ``[B,H_q,T_q,d]`` bf16; k_pages/v_pages ``[num_pages,H_kv,page_size,d]``
    bf16; block_table ``[B,max_pages]`` and kv_lens ``[B]`` int32 on the
    device.  Returns ``o`` (and ``lse`` ``[B,H_q,T_q]`` when ``return_lse``).
    """
    _require_gpu(q)
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H_q, T_q, d], got shape {tuple(q.shape)}")
    B, H_q, T_q, d = q.shape
    dt = _dtype_code(q)
    _check_kv(q, k_pages, v_pages, None)
    num_pages, H_kv, page_size, _ = k_pages.shape
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B={B}, max_pages], got {tuple(block_table.shape)}")
    _expect(block_table, "block_table", None, torch.int32, q.device)
    _expect(kv_lens, "kv_lens", (B,), torch.int32, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, "out", q.shape, q.dtype, q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, H_q, T_q), dtype=torch.float32, device=q.device)
    if return_lse:
        _expect(lse, "lse", (B, H_q, T_q), torch.float32, q.device)
    need = decode_paged_workspace_bytes(B, H_q, H_kv, d, T_q, page_size, max_kv_len,
                                        chunk_tokens, dt)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _expect_workspace(workspace, q.device, need)
    fn = {"both": "gqa_attn_decode_paged", "partial": "gqa_attn_decode_paged_partial",
          "combine": "gqa_attn_decode_paged_combine"}[phase]
    st = getattr(lib(), fn)(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                            _ptr(kv_lens), _ptr(out), _ptr(lse) if return_lse else None,
                            B, H_q, H_kv, d, T_q, page_size, block_table.shape[1],
                            num_pages, int(max_kv_len), scale, dt, chunk_tokens,
                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                            _stream(stream))
    _check(st, fn)
    return (out, lse) if return_lse else out


def merge(o_a, lse_a, o_b, lse_b, out=None, lse_out=None, return_lse=False, stream=None):
    """``gqa_attn_merge`` on torch tensors: stitch two normalised results
    (O ``[..., d]`` and LSE ``[...]`` float32) over disjoint key sets of the
    same query rows.  ``out`` / ``lse_out`` may be the inputs themselves.
    Returns ``o`` (and ``lse`` when ``return_lse``)."""
    _require_gpu(o_a, lse_a, o_b, lse_b)
    if o_a.shape != o_b.shape or lse_a.shape != lse_b.shape or lse_a.shape != o_a.shape[:-1]:
        raise ValueError("o_a, o_b must be [..., d] and lse_a, lse_b their [...] LSEs")
    if o_a.dtype != o_b.dtype or lse_a.dtype != torch.float32 or lse_b.dtype != torch.float32:
        raise TypeError("O inputs share one dtype; LSEs are float32")
    for t, n in ((lse_a, "lse_a"), (o_b, "o_b"), (lse_b, "lse_b")):
        _expect(t, n, None, None, o_a.device)
    d = o_a.shape[-1]
    rows = lse_a.numel()
    if out is None:
        out = torch.empty_like(o_a)
    _expect(out, "out", o_a.shape, o_a.dtype, o_a.device)
    if return_lse and lse_out is None:
        lse_out = torch.empty_like(lse_a)
    if lse_out is not None:
        _expect(lse_out, "lse_out", lse_a.shape, torch.float32, o_a.device)
    st = lib().gqa_attn_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(out),
                              _ptr(lse_out) if (return_lse or lse_out is not None) else None,
                              rows, d, _dtype_code(o_a), _stream(stream))
    _check(st, "gqa_attn_merge")
    return (out, lse_out) if return_lse else out


def prefill(q, k, v, S_kv=None, causal=True, causal_offset=0, scale=None, return_lse=False,
            out=None, lse=None, stream=None):
    """``gqa_attn_prefill`` on torch tensors.

    q ``[B,H_q,S_q,d]``, k/v ``[B,H_kv,kv_cap,d]`` bf16.  ``S_kv`` defaults to
    ``kv_cap``.  Returns ``o`` (and ``lse`` when ``return_lse``).
    """
    _require_gpu(q)
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H_q, S_q, d], got shape {tuple(q.shape)}")
    B, H_q, S_q, d = q.shape
    dt = _dtype_code(q)
    _check_kv(q, k, v, B)
    _, H_kv, kv_cap, _ = k.shape
    S_kv = kv_cap if S_kv is None else int(S_kv)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, "out", q.shape, q.dtype, q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, H_q, S_q), dtype=torch.float32, device=q.device)
    if return_lse:
        _expect(lse, "lse", (B, H_q, S_q), torch.float32, q.device)
    st = lib().gqa_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                _ptr(lse) if return_lse else None, B, H_q, H_kv, d, S_q, S_kv,
                                kv_cap, int(bool(causal)), int(causal_offset), scale, dt,
                                _stream(stream))
    _check(st, "gqa_attn_prefill")
    return (out, lse) if return_lse else out


def prefill_varlen_workspace_bytes(B, H_q, H_kv, max_seqlen_q) -> int:
    return int(lib().gqa_attn_prefill_varlen_workspace_bytes(B, H_q, H_kv, max_seqlen_q))


def prefill_varlen(q, k, v, cu_seqlens_q, kv_lens, max_seqlen_q, max_kv_len=None, causal=True,
                   scale=None, return_lse=False, out=None, lse=None, workspace=None,
                   stream=None):
    """``gqa_attn_prefill_varlen`` on torch tensors.

    q ``[total_q,H_q,d]`` bf16 (sequence b's chunk at rows ``cu_seqlens_q[b]``
    .. ``cu_seqlens_q[b+1]-1``, the newest positions of its cache),
    k/v ``[B,H_kv,kv_cap,d]`` bf16, cu_seqlens_q ``[B+1]`` and kv_lens ``[B]``
    int32 on the device.  ``max_seqlen_q`` bounds every chunk length and
    ``max_kv_len`` (default ``kv_cap``) every cache length: both are host
    values, so no device array is read back.  ``workspace`` (uint8 device
    tensor, allocated when None) holds the work list.  Returns ``o`` (and
    ``lse`` ``[total_q,H_q]`` when ``return_lse``).
    """
    _require_gpu(q)
    if q.dim() != 3:
        raise ValueError(f"q must be [total_q, H_q, d], got shape {tuple(q.shape)}")
    total_q, H_q, d = q.shape
    dt = _dtype_code(q)
    _check_kv(q, k, v, None)
    B, H_kv, kv_cap, _ = k.shape
    _expect(cu_seqlens_q, "cu_seqlens_q", (B + 1,), torch.int32, q.device)
    _expect(kv_lens, "kv_lens", (B,), torch.int32, q.device)
    max_kv_len = kv_cap if max_kv_len is None else int(max_kv_len)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, "out", q.shape, q.dtype, q.device)
    if return_lse and lse is None:
        lse = torch.empty((total_q, H_q), dtype=torch.float32, device=q.device)
    if return_lse:
        _expect(lse, "lse", (total_q, H_q), torch.float32, q.device)
    need = prefill_varlen_workspace_bytes(B, H_q, H_kv, int(max_seqlen_q))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _expect_workspace(workspace, q.device, need)
    st = lib().gqa_attn_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q),
                                       _ptr(kv_lens), _ptr(out),
                                       _ptr(lse) if return_lse else None, B, H_q, H_kv, d,
                                       total_q, int(max_seqlen_q), kv_cap, max_kv_len,
                                       int(bool(causal)), scale, dt, _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(stream))
    _check(st, "gqa_attn_prefill_varlen")
    return (out, lse) if return_lse else out


def prefill_paged(q, k_pages, v_pages, block_table, cu_seqlens_q, kv_lens, max_seqlen_q,
                  max_kv_len=None, causal=True, scale=None, return_lse=False, out=None, lse=None,
                  workspace=None, stream=None):
    """``gqa_attn_prefill_paged`` on torch tensors.

    As :func:`prefill_varlen`, with k_pages/v_pages ``[num_pages,H_kv,page,d]``
    bf16 and block_table ``[B,max_pages]`` int32 on the device; ``max_kv_len``
    defaults to ``max_pages * page``.
    """
    _require_gpu(q)
    if q.dim() != 3:
        raise ValueError(f"q must be [total_q, H_q, d], got shape {tuple(q.shape)}")
    total_q, H_q, d = q.shape
    dt = _dtype_code(q)
    _check_kv(q, k_pages, v_pages, None)
    num_pages, H_kv, page, _ = k_pages.shape
    if block_table.dim() != 2:
        raise ValueError(f"block_table must be [B, max_pages], got {tuple(block_table.shape)}")
    _expect(block_table, "block_table", None, torch.int32, q.device)
    B, max_pages = block_table.shape
    _expect(cu_seqlens_q, "cu_seqlens_q", (B + 1,), torch.int32, q.device)
    _expect(kv_lens, "kv_lens", (B,), torch.int32, q.device)
    max_kv_len = max_pages * page if max_kv_len is None else int(max_kv_len)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, "out", q.shape, q.dtype, q.device)
    if return_lse and lse is None:
        lse = torch.empty((total_q, H_q), dtype=torch.float32, device=q.device)
    if return_lse:
        _expect(lse, "lse", (total_q, H_q), torch.float32, q.device)
    need = prefill_varlen_workspace_bytes(B, H_q, H_kv, int(max_seqlen_q))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _expect_workspace(workspace, q.device, need)
    st = lib().gqa_attn_prefill_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                      _ptr(cu_seqlens_q), _ptr(kv_lens), _ptr(out),
                                      _ptr(lse) if return_lse else None, B, H_q, H_kv, d, total_q,
                                      int(max_seqlen_q), page, max_pages, num_pages, max_kv_len,
                                      int(bool(causal)), scale, dt, _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream))
    _check(st, "gqa_attn_prefill_paged")
    return (out, lse) if return_lse else out
