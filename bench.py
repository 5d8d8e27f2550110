"""Benchmark of the GQA attention hot path on one MI355X.

One step = one pass over both entry points on one batch of synthetic input:
  * decode: Llama3-70B geometry (H_q=64, H_kv=8, d=128), batch 1, 32768 cached
    keys, bf16 (the workload the headline metric is quoted on);
  * prefill: causal, S_q = S_kv = 8192, same geometry, bf16.

``value`` is decode KV throughput in GB/s: algorithmic bytes (K and V of the
valid keys, plus Q and O) per decode call divided by the time per call of K
back-to-back gqa_attn_decode calls, with inputs resident in HBM.  The decode
K/V cache rotates over ``--kv-copies`` distinct copies (default 4 x 128 MiB)
so the 256 MB Infinity Cache cannot serve it from one call to the next.  The
prefill figure (TFLOP/s over the exact causal visible-pair FLOPs) is
reported in the ``prefill`` object.  Each entry point's object carries the
roofline of its main kernel (the decode split kernel, the prefill kernel);
the top-level ``roofline`` repeats the one of the kernel that dominates a
step's GPU time (the prefill kernel in the default run) and says so.

Timing uses HIP events on the stream the kernels run on: around every call
of the K timed steps (decode + prefill), and around the K back-to-back
decode calls and K split-kernel launches that follow; warm-up calls are
untimed.  ``cpu_baseline`` times the fp64 oracle on the host cores on a
bounded sample of the same workload.

After the headline steps, the default run also times the other three
measured workloads -- decode_small_f32 (latency bound), decode_ragged_b4
(HBM bound) and prefill_chunk_64k (matrix-core bound) -- each with its own
roofline object (median and mean), in ``configs``; and a plain device copy
of 1 GiB (``copy_ceiling``: read + write bytes over its median time), the
streaming rate this GPU reaches outside the library, as context for the
spec peak the fractions use.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure (no sparsity)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first (about 0.1 s of work by default: the GPU's clock "
                         "settles within it; a 10-step warm-up measured about 1.5 % lower)")
    ap.add_argument("--kv-copies", type=int, default=4)
    ap.add_argument("--only", choices=["decode", "prefill", "both", "merge"], default="both",
                    help="run one entry point only (for profiler runs); 'merge' times "
                         "gqa_attn_merge stitching two prefill_causal_8k-shaped outputs")
    ap.add_argument("--chunk", type=int, default=0, help="decode keys per split (0 = auto)")
    ap.add_argument("--decode-workload", default="decode_llama70b_32k",
                    help="decode workload name (the headline is decode_llama70b_32k; "
                         "decode_multi_* workloads run gqa_attn_decode_multi)")
    ap.add_argument("--prefill-workload", default="prefill_causal_8k",
                    help="prefill workload name (prefill_varlen_* workloads run "
                         "gqa_attn_prefill_varlen)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of each oracle sample")
    ap.add_argument("--no-fused", action="store_true",
                    help="do not time gqa_attn_decode_fused (a shorter run; its launches "
                         "are decode_fused_bf16_kernel, apart from the two-launch kernels)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other measured workloads and the copy ceiling after the "
                         "headline steps")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device copy 5 times (calibrates the HBM "
                         "byte counters under rocprofv3 --pmc)")
    return ap.parse_args()


def calibrate_copy():
    """Plain device-to-device copy of a known size, for counter calibration."""
    import torch
    n = 512 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": n, "bytes_written": n, "copies": 5}),
          flush=True)


def source_digest(path: str) -> str:
    """First 16 hex digits of the sha256 of a C++/HIP source's code: `//`
    comments (outside string literals) and whitespace removed, so that a
    comment edit leaves it unchanged and any code edit changes it."""
    out, i, text = [], 0, open(path, encoding="utf-8").read()
    in_str = False
    while i < len(text):
        ch = text[i]
        if in_str:
            out.append(ch)
            if ch == "\\":
                out.append(text[i + 1:i + 2])
                i += 2
                continue
            if ch == '"':
                in_str = False
        elif ch == '"':
            in_str = True
            out.append(ch)
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = len(text) if j < 0 else j
            continue
        elif not ch.isspace():
            out.append(ch)
        i += 1
    import hashlib
    return hashlib.sha256("".join(out).encode()).hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary (calibrated FETCH_SIZE + WRITE_SIZE), if it was taken on
    the current kernel source (same code digest); otherwise None."""
    path = os.path.join(ROOT, "profiles", "all_workloads_kernel_stats_and_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    ent = json.loads(m.group(1)).get(f"{kernel}@{workload}")
    if not ent:
        return None
    src = os.path.join(ROOT, "gqa_flashattention_amd", "csrc", ent["source"])
    if source_digest(src) != ent.get("source_code_sha256_16"):
        return None
    return ent["bytes_per_launch"]


GRAPH_KIND = ("the entry point's calls captured in one HIP graph and replayed (median replay / "
              "calls); each replay checked bitwise against an eager call")

TRAFFIC_SOURCE = ("profiles/all_workloads_kernel_stats_and_counters.md: calibrated rocprofv3 "
                  "FETCH_SIZE + WRITE_SIZE per launch, used only when that table was taken on the "
                  "kernel's current source (sha256 of its code, comments and whitespace removed); "
                  "otherwise null")


def measure_copy_ceiling(reps=20):
    """Median time of a plain 1 GiB device-to-device copy (torch copy_):
    (read + write bytes) / time, in GB/s."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    med = ms[len(ms) // 2]
    del dst
    # Read-only streaming: a float32 sum over the same 1 GiB.
    x = src.view(torch.float32)
    for _ in range(3):
        x.sum()
    for a, b in ev:
        a.record(stream)
        x.sum()
        b.record(stream)
    torch.cuda.synchronize()
    rs = sorted(a.elapsed_time(b) for a, b in ev)
    rmed = rs[len(rs) // 2]
    del src, x
    torch.cuda.empty_cache()
    return {"GB_s": round(2 * n / (med * 1e-3) / 1e9, 1), "bytes_read": n, "bytes_written": n,
            "ms_median": round(med, 4), "reps": reps,
            "kind": "torch device-to-device copy of 1 GiB (read + write bytes / median time)",
            "read_only_GB_s": round(n / (rmed * 1e-3) / 1e9, 1),
            "read_only_kind": "torch float32 sum over the same 1 GiB (bytes read / median time)"}


def _stats(ms_list):
    a = sorted(ms_list)
    return sum(a) / len(a), a[len(a) // 2]


def graph_replay_us(call_at, n_calls, out, last_eager, replays=4):
    """Per-call GPU time of `n_calls` calls captured in one HIP graph and
    replayed: median replay time / n_calls, in us.  `call_at(i)` issues call
    i on the current stream (it must allocate nothing).  Before each replay
    `out` is cleared by an eager fill; after it, `out` must equal
    `last_eager()` -- the eager result of the last captured call -- bit for
    bit, or a RuntimeError is raised."""
    import torch
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            for i in range(n_calls):
                call_at(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gms = []
    for r in range(replays):
        out.zero_()
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ga.record()
        g.replay()
        gb.record()
        torch.cuda.synchronize()
        gms.append(ga.elapsed_time(gb))
        want = last_eager()
        torch.cuda.synchronize()
        if not torch.equal(out, want):
            raise RuntimeError(f"graph replay {r} differs from the eager call")
    del g
    return sorted(gms)[len(gms) // 2] * 1e3 / n_calls, len(gms)


def time_decode_workload(name, steps, warmup):
    """Decode workload `name` (gqa_attn_decode): per-call events (median and
    mean), back-to-back calls, and the split kernel alone back to back.
    Caches smaller than 512 MiB rotate over 4 copies (the Infinity Cache
    holds 256 MB)."""
    import torch
    from gqa_flashattention_amd import binding as gq
    from gqa_flashattention_amd import inputs
    w = inputs.WORKLOADS[name]
    dt = gq.DTYPE_F32 if w.dtype == "f32" else gq.DTYPE_BF16
    ncopies = 4 if w.kv_bytes() < (512 << 20) else 1
    copies = [inputs.make_decode(w, device="cuda:0", seed=inputs.SEEDS[name] + 100 * i)
              for i in range(ncopies)]
    # Zero-filled: the fused form's arrival counters start at zero.
    ws = torch.zeros(gq.decode_workspace_bytes(w.B, w.H_q, w.H_kv, w.d, w.max_kv_len, 0, dt),
                     dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(copies[0]["q"])
    stream = torch.cuda.current_stream()

    def call(i, phase="both"):
        x = copies[i % ncopies]
        gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], max_kv_len=w.max_kv_len, scale=w.scale,
                  out=out, workspace=ws, stream=stream, phase=phase)

    for i in range(warmup):
        call(i)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        call(i)
        b.record(stream)
    for i in range(warmup):
        call(i, "fused")
    e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    e[0].record(stream)
    for i in range(steps):
        call(i)
    e[1].record(stream)
    e[2].record(stream)
    for i in range(steps):
        call(i, "partial")
    e[3].record(stream)
    e[4].record(stream)
    for i in range(steps):
        call(i, "fused")
    e[5].record(stream)
    torch.cuda.synchronize()
    mean_ms, med_ms = _stats([a.elapsed_time(b) for a, b in ev])
    b2b_us = e[0].elapsed_time(e[1]) * 1e3 / steps
    part_us = e[2].elapsed_time(e[3]) * 1e3 / steps
    fused_us = e[4].elapsed_time(e[5]) * 1e3 / steps
    graph = None
    if w.kv_bytes() < (16 << 20):
        # A short call is bound by the host's issue rate (about 10 us per
        # call through the binding), not by the GPU: replay `steps` calls
        # captured in one HIP graph to time the GPU side, after checking
        # that a replay reproduces the eager result bit for bit.
        def capture(i):
            x = copies[i % ncopies]
            gq.decode(x["q"], x["k"], x["v"], x["kv_lens"], max_kv_len=w.max_kv_len,
                      scale=w.scale, out=out, workspace=ws)

        def last_eager():
            # The last captured call used copies[(steps - 1) % ncopies].
            last = copies[(steps - 1) % ncopies]
            want = torch.empty_like(out)
            gq.decode(last["q"], last["k"], last["v"], last["kv_lens"], max_kv_len=w.max_kv_len,
                      scale=w.scale, out=want, workspace=torch.empty_like(ws))
            return want

        g_us, reps = graph_replay_us(capture, steps, out, last_eager)
        graph = {"us_per_call": round(g_us, 3), "calls_per_graph": steps, "replays": reps,
                 "kind": GRAPH_KIND}
    gbs = w.decode_bytes() / (b2b_us * 1e-6) / 1e9
    part_bytes = w.kv_bytes() + w.B * w.H_q * w.T_q * w.d * w.elem_bytes
    part_gbs = part_bytes / (part_us * 1e-6) / 1e9
    res = {"entry_point": "gqa_attn_decode", "B": w.B, "kv_lens": list(w.lens), "dtype": w.dtype,
           "kv_copies": ncopies, "keys_per_split": gq.decode_split_tokens(w.B, w.H_kv,
                                                                        w.max_kv_len, 0, dt),
           "us_per_call_back_to_back": round(b2b_us, 3),
           "us_per_call_median": round(med_ms * 1e3, 3), "us_per_call_mean": round(mean_ms * 1e3, 3),
           "bytes_per_call": w.decode_bytes(), "GB_s": round(gbs, 2),
           "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
           "fused": {"entry_point": "gqa_attn_decode_fused",
                     "us_per_call_back_to_back": round(fused_us, 3),
                     "GB_s": round(w.decode_bytes() / (fused_us * 1e-6) / 1e9, 2)},
           "graph_replay": graph,
           "roofline": {"bound": "hbm" if w.dtype == "bf16" else "latency",
                        "kernel": f"decode_partial_{w.dtype}_kernel",
                        "achieved": round(part_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(part_gbs / HBM_PEAK_GBS, 4),
                        "traffic": traffic_from_profiles("decode_partial", name),
                        "traffic_source": TRAFFIC_SOURCE,
                        "algorithmic_bytes_per_launch": part_bytes,
                        "launch_us_mean": round(part_us, 3)}}
    del copies, ws, out
    torch.cuda.empty_cache()
    return res


def time_prefill_workload(name, steps, warmup):
    """Prefill workload `name` (gqa_attn_prefill): per-call events, TFLOP/s
    of the median and of the mean call."""
    import torch
    from gqa_flashattention_amd import binding as gq
    from gqa_flashattention_amd import inputs
    w = inputs.WORKLOADS[name]
    x = inputs.make_prefill(w, device="cuda:0")
    out = torch.empty_like(x["q"])
    stream = torch.cuda.current_stream()

    def call():
        gq.prefill(x["q"], x["k"], x["v"], S_kv=w.S_kv, causal=w.causal, causal_offset=w.offset,
                   scale=w.scale, out=out, stream=stream)

    for _ in range(warmup):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    mean_ms, med_ms = _stats([a.elapsed_time(b) for a, b in ev])
    tf_med = w.prefill_flops() / (med_ms * 1e-3) / 1e12
    tf_mean = w.prefill_flops() / (mean_ms * 1e-3) / 1e12
    res = {"entry_point": "gqa_attn_prefill", "S_q": w.S_q, "S_kv": w.S_kv, "offset": w.offset,
           "causal": w.causal, "ms_median": round(med_ms, 6), "ms_mean": round(mean_ms, 6),
           "flops_per_call": w.prefill_flops(), "TFLOP_s": round(tf_med, 2),
           "TFLOP_s_mean": round(tf_mean, 2),
           "roofline": {"bound": "mfma", "kernel": "prefill_bf16_kernel<false, false>",
                        "achieved": round(tf_med, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf_med / BF16_PEAK_TFLOPS, 4),
                        "frac_mean": round(tf_mean / BF16_PEAK_TFLOPS, 4),
                        "traffic": traffic_from_profiles("prefill", name),
                        "traffic_source": TRAFFIC_SOURCE,
                        "launch_us_median": round(med_ms * 1e3, 3),
                        "launch_us_mean": round(mean_ms * 1e3, 3)}}
    del x, out
    torch.cuda.empty_cache()
    return res


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        return int(n)
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline_decode(w, x_cpu, seconds):
    """Oracle over whole decode calls of the workload, repeated to ~seconds."""
    import numpy as np
    import oracle
    lens = np.array(w.lens)
    if w.kind == "decode_paged":
        args = (x_cpu["q"], x_cpu["k_pages"], x_cpu["v_pages"], x_cpu["block_table"], lens,
                w.page_size, w.scale)
        fn = oracle.decode_paged
    else:
        args = (x_cpu["q"], x_cpu["k"], x_cpu["v"], lens, w.scale)
        fn = oracle.decode_multi if w.kind == "decode_multi" else oracle.decode
    reps, t0 = 0, time.perf_counter()
    while True:
        fn(*args)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    gbs = w.decode_bytes() * reps / el / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{reps} full decode call(s) of {w.name} (B={w.B}, lens={list(w.lens)}, "
                      f"T_q={w.T_q}, all {w.H_q} heads) in {el:.1f} s, numpy fp64"}


def cpu_baseline_prefill(w, x_cpu, seconds):
    """Oracle on a seeded sample of query rows (all 64 heads), rows added in
    blocks until ~seconds of CPU time; FLOPs counted exactly per row."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(7)
    order = rng.permutation(w.S_q)
    q, k, v = (x_cpu[n] for n in ("q", "k", "v"))
    done, flops, t0 = 0, 0, time.perf_counter()
    while done < w.S_q:
        rows = np.sort(order[done:done + 64])
        oracle.prefill(q, k, v, w.S_kv, w.scale, causal=w.causal, causal_offset=w.offset,
                       rows=rows)
        vis = oracle.prefill_visible_len(rows, w.S_kv, w.causal, w.offset)
        flops += 4 * w.d * w.H_q * w.B * int(vis.sum())
        done += len(rows)
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": cpu_threads(),
            "kind": "oracle",
            "sample": f"{done} seeded query rows x {w.H_q} heads of {w.name} in {el:.1f} s, "
                      f"numpy fp64"}


def cpu_baseline_prefill_varlen(w, x_cpu, seconds):
    """Oracle on seeded query rows of every chunk of a varlen batch (all 64
    heads), taken round-robin over the sequences in blocks of up to 16 rows
    until ~seconds of CPU time; FLOPs counted exactly per row."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(7)
    cu = np.concatenate([[0], np.cumsum(w.q_lens)])
    orders = [rng.permutation(sq) for sq in w.q_lens]
    q, k, v = (x_cpu[n] for n in ("q", "k", "v"))
    done, flops, pos, t0 = 0, 0, [0] * w.B, time.perf_counter()
    while time.perf_counter() - t0 < seconds and done < w.total_q:
        for b, (sq, L) in enumerate(zip(w.q_lens, w.lens)):
            if pos[b] >= sq:
                continue
            rows = np.sort(orders[b][pos[b]:pos[b] + 16])
            pos[b] += len(rows)
            qb = np.transpose(q[cu[b]:cu[b + 1]], (1, 0, 2))[None]
            oracle.prefill(qb, k[b:b + 1], v[b:b + 1], L, w.scale, causal=w.causal,
                           causal_offset=L - sq, rows=rows)
            vis = oracle.prefill_visible_len(rows, L, w.causal, L - sq)
            flops += 4 * w.d * w.H_q * int(vis.sum())
            done += len(rows)
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": cpu_threads(),
            "kind": "oracle",
            "sample": f"{done} seeded query rows (up to 16 per chunk per round) x {w.H_q} heads "
                      f"of {w.name} in {el:.1f} s, numpy fp64"}


def bench_merge(args):
    """gqa_attn_merge on two results of the prefill_causal_8k shape: rows =
    64 heads x 8192 positions, O bf16 [rows, 128], LSE float32.  HBM bound:
    reads 2 x (O + LSE), writes O + LSE."""
    import torch
    from gqa_flashattention_amd import binding as gq
    rows, d = 64 * 8192, 128
    g = torch.Generator(device="cuda:0").manual_seed(20260099)
    mk = lambda: torch.randn(rows, d, device="cuda:0", generator=g).to(torch.bfloat16)
    oa, ob = mk(), mk()
    la = torch.randn(rows, device="cuda:0", generator=g) * 3
    lb = torch.randn(rows, device="cuda:0", generator=g) * 3
    out, lout = torch.empty_like(oa), torch.empty_like(la)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        gq.merge(oa, la, ob, lb, out=out, lse_out=lout, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        gq.merge(oa, la, ob, lb, out=out, lse_out=lout, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    nbytes = 3 * rows * d * 2 + 3 * rows * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    out_line = {
        "metric": "decode KV GB/s (% HBM peak); causal prefill TFLOP/s (% bf16 MFMA peak)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "merge_prefill_8k (gqa_attn_merge)", "rows": rows, "d": d},
        "roofline": {"bound": "hbm", "kernel": "merge_kernel<bf16>", "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profiles("merge", "merge_prefill_8k"),
                     "algorithmic_bytes_per_launch": nbytes, "launch_us_mean": round(us, 3)},
    }
    print(json.dumps(out_line), flush=True)


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not "
              "supported (the multi-GPU sharding is described, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    from gqa_flashattention_amd import binding as gq
    from gqa_flashattention_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.only == "merge":
        bench_merge(args)
        return

    wd = inputs.WORKLOADS[args.decode_workload]
    dec_dtype = gq.DTYPE_F32 if wd.dtype == "f32" else gq.DTYPE_BF16
    multi = wd.kind in ("decode_multi", "decode_paged")
    paged = wd.kind == "decode_paged"
    wp = inputs.WORKLOADS[args.prefill_workload]
    varlen = wp.kind in ("prefill_varlen", "prefill_paged")
    paged_pre = wp.kind == "prefill_paged"
    do_dec = args.only in ("decode", "both")
    do_pre = args.only in ("prefill", "both")

    # ---- inputs, resident in HBM before timing
    if do_dec:
        if paged:
            make = lambda w, device, seed: inputs.make_decode_paged(w, w.page_size, device=device,
                                                                    seed=seed)
        else:
            make = inputs.make_decode_multi if multi else inputs.make_decode
        copies = [make(wd, device=dev, seed=inputs.SEEDS[wd.name] + 100 * i)
                  for i in range(max(1, args.kv_copies))]
        if paged:
            need = gq.decode_paged_workspace_bytes(wd.B, wd.H_q, wd.H_kv, wd.d, wd.T_q,
                                                   wd.page_size, wd.max_kv_len, args.chunk,
                                                   dec_dtype)
            chunk = gq.decode_paged_split_tokens(wd.B, wd.H_q, wd.H_kv, wd.T_q, wd.page_size,
                                                 wd.max_kv_len, args.chunk, dec_dtype)
            for x in copies:          # only the pages are read; drop the contiguous copy
                del x["k"], x["v"]
        elif multi:
            need = gq.decode_multi_workspace_bytes(wd.B, wd.H_q, wd.H_kv, wd.d, wd.T_q,
                                                   wd.max_kv_len, args.chunk, dec_dtype)
            chunk = gq.decode_multi_split_tokens(wd.B, wd.H_q, wd.H_kv, wd.T_q, wd.max_kv_len,
                                                 args.chunk, dec_dtype)
        else:
            need = gq.decode_workspace_bytes(wd.B, wd.H_q, wd.H_kv, wd.d, wd.max_kv_len,
                                             args.chunk, dec_dtype)
            chunk = gq.decode_split_tokens(wd.B, wd.H_kv, wd.max_kv_len, args.chunk, dec_dtype)
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)   # fused counters start at zero
        o_dec = torch.empty_like(copies[0]["q"])
    if do_pre:
        if paged_pre:
            # The contiguous k, v it was scattered from stay for the oracle leg.
            xp = inputs.make_prefill_paged(wp, wp.page_size, device=dev)
        else:
            xp = (inputs.make_prefill_varlen if varlen else inputs.make_prefill)(wp, device=dev)
        o_pre = torch.empty_like(xp["q"])
    torch.cuda.synchronize()

    def prefill_call():
        if paged_pre:
            gq.prefill_paged(xp["q"], xp["k_pages"], xp["v_pages"], xp["block_table"],
                             xp["cu_seqlens_q"], xp["kv_lens"], max_seqlen_q=max(wp.q_lens),
                             max_kv_len=wp.max_kv_len, causal=wp.causal, scale=wp.scale,
                             out=o_pre, stream=stream)
            return
        if varlen:
            gq.prefill_varlen(xp["q"], xp["k"], xp["v"], xp["cu_seqlens_q"], xp["kv_lens"],
                              max_seqlen_q=max(wp.q_lens), max_kv_len=wp.max_kv_len,
                              causal=wp.causal, scale=wp.scale, out=o_pre, stream=stream)
            return
        gq.prefill(xp["q"], xp["k"], xp["v"], S_kv=wp.S_kv, causal=wp.causal,
                   causal_offset=wp.offset, scale=wp.scale, out=o_pre, stream=stream)

    def decode_call(i, phase="both", on=None, out=None, wsp=None):
        # on=None: the timing stream; a graph capture passes the capturing one.
        x = copies[i % len(copies)]
        st = stream if on is None else on
        o = o_dec if out is None else out
        w_ = ws if wsp is None else wsp
        if paged:
            gq.decode_paged(x["q"], x["k_pages"], x["v_pages"], x["block_table"], x["kv_lens"],
                            max_kv_len=wd.max_kv_len, scale=wd.scale, chunk_tokens=args.chunk,
                            out=o, workspace=w_, stream=st, phase=phase)
            return
        fn = gq.decode_multi if multi else gq.decode
        fn(x["q"], x["k"], x["v"], x["kv_lens"], max_kv_len=wd.max_kv_len,
           scale=wd.scale, chunk_tokens=args.chunk, out=o, workspace=w_,
           stream=st, phase=phase)

    for i in range(args.warmup):
        if do_dec:
            decode_call(i)
        if do_pre:
            prefill_call()
    torch.cuda.synchronize()

    # Timed region.
    #  (1) K steps: one gqa_attn_decode call and one prefill call each, HIP
    #      events around every call (ms_per_step; the prefill figure).
    #  (2) K gqa_attn_decode calls back to back (rotating K/V copies) between
    #      two events: the decode throughput, `value`.  Per-call events would
    #      add their own overhead to a ~30 us call.
    #  (3) K launches of the decode split kernel alone
    #      (gqa_attn_decode_partial) between two events: its per-launch
    #      duration, for the roofline.
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    kd = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    kp = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    kf = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    fused_ok = do_dec and not multi and not paged and not args.no_fused
    if fused_ok:
        for i in range(min(args.warmup, 20)):
            decode_call(i, "fused")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        if do_dec:
            decode_call(i)
        ev[i][1].record(stream)
        if do_pre:
            prefill_call()
        ev[i][2].record(stream)
    if do_dec:
        kd[0].record(stream)
        for i in range(K):
            decode_call(i)
        kd[1].record(stream)
        kp[0].record(stream)
        for i in range(K):
            decode_call(i, "partial")
        kp[1].record(stream)
        if fused_ok:
            kf[0].record(stream)
            for i in range(K):
                decode_call(i, "fused")
            kf[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    dec_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]
    pre_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]
    step_ms = [ev[i][0].elapsed_time(ev[i][2]) for i in range(K)]
    dec_b2b_us = kd[0].elapsed_time(kd[1]) * 1e3 / K if do_dec else None
    part_us = kp[0].elapsed_time(kp[1]) * 1e3 / K if do_dec else None
    # (4) The same K back-to-back decode calls captured in one HIP graph and
    #     replayed (context beside `value`, which stays the eager rate).
    dec_graph = None
    if do_dec:
        def last_eager():
            want = torch.empty_like(o_dec)
            decode_call(K - 1, out=want, wsp=torch.empty_like(ws))
            return want
        g_us, reps = graph_replay_us(lambda i: decode_call(i, on=torch.cuda.current_stream()),
                                     K, o_dec, last_eager)
        dec_graph = {"us_per_call": round(g_us, 3), "calls_per_graph": K, "replays": reps,
                     "GB_s": round(wd.decode_bytes() / (g_us * 1e-6) / 1e9, 2),
                     "kind": GRAPH_KIND}
    mean = lambda a: sum(a) / len(a)
    median = lambda a: sorted(a)[len(a) // 2]

    out = {
        "metric": "decode KV GB/s (% HBM peak); causal prefill TFLOP/s (% bf16 MFMA peak)",
        "value": None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(mean(step_ms), 6),
        "ms_per_step_median": round(median(step_ms), 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wd.dtype if args.only == "decode" else "bf16",
        "data": "synthetic",
        "config": {"workload": " + ".join(n for n, on in ((wd.name, do_dec), (wp.name, do_pre)) if on),
                   "decode": {"B": wd.B, "H_q": wd.H_q, "H_kv": wd.H_kv, "d": wd.d,
                              "T_q": wd.T_q, "page_size": wd.page_size or None,
                              "entry_point": "gqa_attn_decode_paged" if paged else
                              "gqa_attn_decode_multi" if multi else "gqa_attn_decode",
                              "kv_lens": list(wd.lens), "kv_copies": len(copies) if do_dec else 0,
                              "keys_per_split": chunk if do_dec else None},
                   "prefill": ({"B": wp.B, "H_q": wp.H_q, "H_kv": wp.H_kv, "d": wp.d,
                                "entry_point": "gqa_attn_prefill_paged" if paged_pre else
                                "gqa_attn_prefill_varlen", "page_size": wp.page_size or None,
                                "q_lens": list(wp.q_lens), "kv_lens": list(wp.lens),
                                "causal": wp.causal} if varlen else
                               {"B": wp.B, "H_q": wp.H_q, "H_kv": wp.H_kv, "d": wp.d,
                                "S_q": wp.S_q, "S_kv": wp.S_kv, "causal": wp.causal,
                                "offset": wp.offset})},
        "wall_s_timed_region": round(wall, 4),
    }
    if do_dec:
        t_s = dec_b2b_us / 1e6
        gbs = wd.decode_bytes() / t_s / 1e9
        # Split kernel's algorithmic bytes: K and V of the valid keys plus Q.
        part_bytes = wd.kv_bytes() + wd.B * wd.H_q * wd.T_q * wd.d * wd.elem_bytes
        part_gbs = part_bytes / (part_us / 1e6) / 1e9
        out["value"] = round(gbs, 2)
        out["decode"] = {"us_per_call_back_to_back": round(dec_b2b_us, 3),
                         "ms_mean_in_step": round(mean(dec_ms), 6),
                         "ms_median_in_step": round(median(dec_ms), 6),
                         "GB_s": round(gbs, 2), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                         "bytes_per_call": wd.decode_bytes(),
                         "partial_kernel_us_mean": round(part_us, 3),
                         "graph_replay": dec_graph}
        if fused_ok:
            f_us = kf[0].elapsed_time(kf[1]) * 1e3 / K
            out["decode"]["fused"] = {"entry_point": "gqa_attn_decode_fused",
                                      "us_per_call_back_to_back": round(f_us, 3),
                                      "GB_s": round(wd.decode_bytes() / (f_us * 1e-6) / 1e9, 2)}
        if multi and wd.G * wd.T_q > 16:
            rows = wd.G * wd.T_q
            rgroups = 1 if rows <= 32 else (2 if rows <= 64 else 4)
            kname, tkey = f"decode_multi_partial_kernel<{rgroups}>", "decode_multi_partial"
            tf = wd.decode_multi_flops() / t_s / 1e12
            out["decode"].update({"flops_per_call": wd.decode_multi_flops(),
                                  "TFLOP_s": round(tf, 3),
                                  "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)})
        else:
            kname, tkey = f"decode_partial_{wd.dtype}_kernel", "decode_partial"
        out["decode"]["roofline"] = {"bound": "hbm", "kernel": kname,
                                     "achieved": round(part_gbs, 2), "peak": HBM_PEAK_GBS,
                                     "unit": "GB/s", "frac": round(part_gbs / HBM_PEAK_GBS, 4),
                                     "traffic": traffic_from_profiles(tkey, wd.name),
                                     "traffic_source": TRAFFIC_SOURCE,
                                     "algorithmic_bytes_per_launch": part_bytes,
                                     "launch_us_mean": round(part_us, 3)}
    if do_pre:
        # The median call is the reported figure; the mean is given beside it.
        tf = wp.prefill_flops() / (median(pre_ms) / 1e3) / 1e12
        tf_mean = wp.prefill_flops() / (mean(pre_ms) / 1e3) / 1e12
        out["prefill"] = {"value": round(tf, 2), "unit": "TFLOP/s",
                          "value_of_mean_call": round(tf_mean, 2),
                          "ms_mean": round(mean(pre_ms), 6), "ms_median": round(median(pre_ms), 6),
                          "flops_per_call": wp.prefill_flops(),
                          "roofline": {"bound": "mfma",
                                       "kernel": f"prefill_bf16_kernel<{str(varlen).lower()}, "
                                                 f"{str(paged_pre).lower()}>",
                                       "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                                       "frac_mean": round(tf_mean / BF16_PEAK_TFLOPS, 4),
                                       "traffic": traffic_from_profiles("prefill", wp.name),
                                       "traffic_source": TRAFFIC_SOURCE,
                                       "launch_us_median": round(median(pre_ms) * 1e3, 3),
                                       "launch_us_mean": round(mean(pre_ms) * 1e3, 3)}}

    if not do_dec:   # prefill-only run: its throughput is the value
        out["value"] = out["prefill"]["value"]
        out["unit"] = "TFLOP/s"
    # The top-level roofline is that of the kernel that dominates one step's
    # GPU time (each entry point's object keeps its own).
    shares = {}
    if do_dec:
        shares["decode"] = median(dec_ms)
    if do_pre:
        shares["prefill"] = median(pre_ms)
    dom = max(shares, key=shares.get)
    out["roofline"] = dict(out[dom]["roofline"])
    out["roofline"]["dominant_in_step"] = (
        f"{dom}: {shares[dom] * 1e3:.1f} of the step's {sum(shares.values()) * 1e3:.1f} us "
        f"(median calls, HIP events)")

    # The other measured workloads and the copy ceiling, after the headline
    # (default run only: the headline workloads and both entry points).
    default_run = (args.only == "both" and args.decode_workload == "decode_llama70b_32k"
                   and args.prefill_workload == "prefill_causal_8k" and args.chunk == 0)
    if default_run and not args.no_extra:
        del copies, ws, xp, o_dec, o_pre
        torch.cuda.empty_cache()
        cfg = {}
        for name in ("decode_small_f32", "decode_ragged_b4"):
            cfg[name] = time_decode_workload(name, K, max(args.warmup, 10))
        cfg["prefill_chunk_64k"] = time_prefill_workload("prefill_chunk_64k", min(K, 20),
                                                         min(max(args.warmup // 10, 3), 10))
        out["configs"] = cfg
        out["copy_ceiling"] = measure_copy_ceiling()
        if not args.no_cpu_baseline:
            # Re-create the headline inputs for the oracle leg (same seeds).
            copies = [inputs.make_decode(wd, device=dev, seed=inputs.SEEDS[wd.name])]
            xp = inputs.make_prefill(wp, device=dev)

    if not args.no_cpu_baseline:
        import numpy as np  # noqa: F401
        if do_dec:
            names = ("q", "k_pages", "v_pages", "block_table") if paged else ("q", "k", "v")
            xc = {n: (copies[0][n].cpu().numpy() if n == "block_table"
                      else copies[0][n].float().cpu().numpy()) for n in names}
            out["cpu_baseline"] = cpu_baseline_decode(wd, xc, args.cpu_seconds)
            del xc
        if do_pre:
            xc = {n: xp[n].float().cpu().numpy() for n in ("q", "k", "v")}
            fn = cpu_baseline_prefill_varlen if varlen else cpu_baseline_prefill
            out["prefill"]["cpu_baseline"] = fn(wp, xc, args.cpu_seconds)
            del xc

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
