"""HIP-graph capture of the entry points: a call captured once and replayed
with new inputs copied into its buffers gives, on every replay, exactly the
result of an eager call on those inputs.

Each entry point allocates nothing inside the captured call (outputs, LSE
buffers and workspaces are passed in), clears nothing with a memset, and
reads its inputs only through the pointers it was given, so a replay sees
whatever the buffers hold at replay time.  Between replays the test does
eager work (the copies of the next inputs, a synchronisation)."""

import pytest
import torch

from gpu_util import banner
from gqa_flashattention_amd import binding as gq
from gqa_flashattention_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _capture(call):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def _replays_match(static, sets, call, outs):
    """`static`: dict of input buffers; `sets`: list of dicts of inputs of
    the same shapes; `call()` runs the entry point on `static` into `outs`.
    Eager results per set first, then one capture and a replay per set."""
    want = []
    for x in sets:
        for k, t in static.items():
            t.copy_(x[k])
        call()
        torch.cuda.synchronize()
        want.append([o.clone() for o in outs])
    g = _capture(call)
    for r, x in enumerate(sets):
        for o in outs:
            o.fill_(float("nan")) if o.is_floating_point() else o.zero_()
        for k, t in static.items():
            t.copy_(x[k])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want[r]):
            assert torch.equal(o, w), f"replay {r} differs from the eager call"
    del g


def test_graph_decode_two_launches():
    w = inputs.Workload("t", "decode", B=2, H_q=64, H_kv=8, d=128, dtype="bf16", lens=(3000, 1234),
                        kv_cap=3000)
    banner("graph_decode", w.lens)
    sets = [inputs.make_decode(w, device=DEV, seed=90 + i) for i in range(3)]
    static = {k: sets[0][k].clone() for k in ("q", "k", "v", "kv_lens")}
    ws = torch.empty(gq.decode_workspace_bytes(2, 64, 8, 128, 3000, 0, gq.DTYPE_BF16), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty_like(static["q"])
    lse = torch.empty((2, 64), dtype=torch.float32, device=DEV)
    call = lambda: gq.decode(static["q"], static["k"], static["v"], static["kv_lens"], max_kv_len=3000,
                             scale=w.scale, out=out, lse=lse, return_lse=True, workspace=ws)
    _replays_match(static, sets, call, [out, lse])


def test_graph_decode_multi_and_fp32():
    w = inputs.Workload("t", "decode_multi", B=1, H_q=64, H_kv=8, d=128, dtype="bf16", lens=(2500,),
                        kv_cap=2500, T_q=4)
    banner("graph_decode_multi", w.lens, w.T_q)
    sets = [inputs.make_decode_multi(w, device=DEV, seed=95 + i) for i in range(3)]
    static = {k: sets[0][k].clone() for k in ("q", "k", "v", "kv_lens")}
    ws = torch.empty(gq.decode_multi_workspace_bytes(1, 64, 8, 128, 4, 2500, 0, gq.DTYPE_BF16),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(static["q"])
    call = lambda: gq.decode_multi(static["q"], static["k"], static["v"], static["kv_lens"], max_kv_len=2500,
                                   scale=w.scale, out=out, workspace=ws)
    _replays_match(static, sets, call, [out])

    w32 = inputs.WORKLOADS["decode_small_f32"]
    banner("graph_decode_f32", w32.name)
    sets = [inputs.make_decode(w32, device=DEV, seed=98 + i) for i in range(3)]
    static = {k: sets[0][k].clone() for k in ("q", "k", "v", "kv_lens")}
    ws = torch.empty(gq.decode_workspace_bytes(1, 8, 1, 128, 256, 0, gq.DTYPE_F32), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty_like(static["q"])
    call = lambda: gq.decode(static["q"], static["k"], static["v"], static["kv_lens"], max_kv_len=256,
                             scale=w32.scale, out=out, workspace=ws)
    _replays_match(static, sets, call, [out])


def test_graph_prefill():
    w = inputs.Workload("t", "prefill", B=1, H_q=16, H_kv=2, d=128, dtype="bf16", S_q=700, S_kv=700)
    banner("graph_prefill", w.S_q)
    sets = [inputs.make_prefill(w, device=DEV, seed=101 + i) for i in range(3)]
    static = {k: sets[0][k].clone() for k in ("q", "k", "v")}
    out = torch.empty_like(static["q"])
    lse = torch.empty(static["q"].shape[:3], dtype=torch.float32, device=DEV)
    call = lambda: gq.prefill(static["q"], static["k"], static["v"], S_kv=700, causal=True, scale=w.scale,
                              out=out, lse=lse, return_lse=True)
    _replays_match(static, sets, call, [out, lse])
