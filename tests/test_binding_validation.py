"""The Python binding rejects mismatched tensors on the host, before any
pointer reaches the library (CPU only).

Every wrapper checks that K and V have q's dtype, device and head dimension,
that batch sizes agree, and that caller-supplied outputs, LSE buffers and
workspaces have the right shape, dtype, device, contiguity and size.  Here
the GPU-residency check is disabled and the library is replaced by a stub
whose sizing queries forward to the real library and whose compute entry
points fail the test if reached, so a missing check shows up as a failure
instead of a launch."""

import os

import pytest
import torch

from gqa_flashattention_amd import binding

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libgqa_attn.so not built")


class _StubLib:
    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name.endswith(("_bytes", "_split_tokens", "status_string")):
            return getattr(self._real, name)

        def reached(*a):
            raise AssertionError(f"{name} reached the library: a host check is missing")
        return reached


@pytest.fixture(autouse=True)
def _host_only(monkeypatch):
    real = binding.lib()
    monkeypatch.setattr(binding, "_require_gpu", lambda *ts: None)
    monkeypatch.setattr(binding, "lib", lambda: _StubLib(real))


bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32


def _t(shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def _dec(**over):
    a = dict(q=_t((2, 16, 128)), k=_t((2, 2, 64, 128)), v=_t((2, 2, 64, 128)),
             kv_lens=_t((2,), i32))
    a.update(over)
    return a


@pytest.mark.parametrize("over,exc", [
    (dict(k=_t((2, 2, 64, 128), f32), v=_t((2, 2, 64, 128), f32)), TypeError),   # bf16 q, f32 cache
    (dict(q=_t((2, 16, 128), f32)), TypeError),                                 # f32 q, bf16 cache
    (dict(v=_t((2, 2, 32, 128))), ValueError),                                  # V shorter than K
    (dict(k=_t((1, 2, 64, 128)), v=_t((1, 2, 64, 128))), ValueError),           # fewer sequences
    (dict(k=_t((2, 2, 64, 64)), v=_t((2, 2, 64, 64))), ValueError),             # other d
    (dict(kv_lens=_t((3,), i32)), ValueError),
    (dict(kv_lens=_t((2,), torch.int64)), TypeError),
    (dict(k=_t((2, 2, 128, 64)).transpose(2, 3)), ValueError),                  # strided K
])
def test_decode_rejects_mismatched_inputs(over, exc):
    a = _dec(**over)
    with pytest.raises(exc):
        binding.decode(a["q"], a["k"], a["v"], a["kv_lens"])


@pytest.mark.parametrize("kw,exc", [
    (dict(out=_t((2, 16, 64))), ValueError),
    (dict(out=_t((2, 16, 128), f32)), TypeError),
    (dict(out=_t((2, 128, 16)).transpose(1, 2)), ValueError),
    (dict(return_lse=True, lse=_t((2, 8), f32)), ValueError),
    (dict(return_lse=True, lse=_t((2, 16), bf)), TypeError),
    (dict(workspace=_t((16,), torch.uint8)), ValueError),                        # too small
    (dict(workspace=_t((1 << 20,), torch.uint8)[::2]), ValueError),              # strided
])
def test_decode_rejects_bad_outputs_and_workspace(kw, exc):
    a = _dec()
    with pytest.raises(exc):
        binding.decode(a["q"], a["k"], a["v"], a["kv_lens"], **kw)


def test_decode_multi_and_paged_checks():
    q = _t((2, 16, 4, 128))
    k = _t((2, 2, 64, 128))
    lens = _t((2,), i32)
    with pytest.raises(TypeError):
        binding.decode_multi(q, k.float(), k.float(), lens)
    with pytest.raises(ValueError):
        binding.decode_multi(q, k[:1].contiguous(), k[:1].contiguous(), lens)
    with pytest.raises(ValueError):
        binding.decode_multi(q, k, k, lens, return_lse=True, lse=_t((2, 16, 2), f32))
    pages = _t((10, 2, 16, 128))
    table = _t((2, 4), i32)
    with pytest.raises(TypeError):
        binding.decode_paged(q, pages, pages.float(), table, lens, max_kv_len=64)
    with pytest.raises(ValueError):
        binding.decode_paged(q, pages, pages, _t((3, 4), i32), lens, max_kv_len=64)
    with pytest.raises(TypeError):
        binding.decode_paged(q, pages, pages, table.long(), lens, max_kv_len=64)
    with pytest.raises(ValueError):
        binding.decode_paged(q, pages, pages[:, :, :8].contiguous(), table, lens, max_kv_len=64)


def test_prefill_checks():
    q = _t((1, 16, 64, 128))
    k = _t((1, 2, 64, 128))
    with pytest.raises(TypeError):
        binding.prefill(q, k.float(), k.float())
    with pytest.raises(ValueError):
        binding.prefill(q, k, _t((1, 2, 48, 128)))
    with pytest.raises(ValueError):
        binding.prefill(q, _t((2, 2, 64, 128)), _t((2, 2, 64, 128)))
    with pytest.raises(ValueError):
        binding.prefill(q, k, k, out=_t((1, 16, 32, 128)))
    with pytest.raises(ValueError):
        binding.prefill(q, k, k, return_lse=True, lse=_t((1, 16, 32), f32))
    with pytest.raises(ValueError):
        binding.prefill(_t((16, 64, 128)), k, k)


def test_prefill_varlen_and_paged_checks():
    q = _t((100, 16, 128))
    k = _t((3, 2, 64, 128))
    cu = _t((4,), i32)
    lens = _t((3,), i32)
    with pytest.raises(TypeError):
        binding.prefill_varlen(q, k, k.float(), cu, lens, max_seqlen_q=64)
    with pytest.raises(ValueError):
        binding.prefill_varlen(q, k, k, _t((3,), i32), lens, max_seqlen_q=64)
    with pytest.raises(ValueError):
        binding.prefill_varlen(q, k, k, cu, lens, max_seqlen_q=64, out=_t((99, 16, 128)))
    with pytest.raises(ValueError):
        binding.prefill_varlen(q, k, k, cu, lens, max_seqlen_q=64,
                               workspace=_t((4,), torch.uint8))
    pages = _t((20, 2, 16, 128))
    table = _t((3, 4), i32)
    with pytest.raises(TypeError):
        binding.prefill_paged(q, pages, pages, table, cu, lens.long(), max_seqlen_q=64)
    with pytest.raises(ValueError):
        binding.prefill_paged(q, pages, pages, table, _t((5,), i32), lens, max_seqlen_q=64)
    with pytest.raises(TypeError):
        binding.prefill_paged(q, pages.float(), pages.float(), table, cu, lens, max_seqlen_q=64)


def test_merge_checks():
    o = _t((32, 128))
    l = _t((32,), f32)
    with pytest.raises(ValueError):
        binding.merge(o, l, o, l, out=_t((32, 64)))
    with pytest.raises(TypeError):
        binding.merge(o, l, o, l, out=_t((32, 128), f32))
    with pytest.raises(ValueError):
        binding.merge(o, l, o, l, lse_out=_t((16,), f32))
    with pytest.raises(TypeError):
        binding.merge(o, l, o.float(), l)
