"""bench.py's output contract: one JSON line with the fields the round-end
measurement reads, and the one-GPU guard.

The GPU case runs a short bench (a few steps, no CPU baseline, no extra
workloads) in a child process and checks the fields and their consistency;
the figures themselves are not judged here."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")

TOP_KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
            "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline"}
ROOFLINE_KEYS = {"bound", "kernel", "achieved", "peak", "unit", "frac", "traffic", "traffic_source"}


def test_more_than_one_gpu_is_refused():
    """--gpus N > 1 exits with status 2 and says why, before touching a GPU."""
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_source_digest_follows_code_not_comments(tmp_path):
    """roofline.traffic is reused only while the kernel's code is unchanged:
    the digest ignores `//` comments and whitespace, not code or string
    contents (a `//` inside a string literal is code)."""
    sys.path.insert(0, ROOT)
    import bench
    a, b, c, d = (tmp_path / n for n in ("a.hip", "b.hip", "c.hip", "d.hip"))
    a.write_text('int x = 1;  // one\n  asm("s_nop // a \\" b");\n')
    b.write_text('// header\nint x = 1;\nasm("s_nop // a \\" b"); // trailing\n')
    c.write_text('int x = 2;\nasm("s_nop // a \\" b");\n')
    d.write_text('int x = 1;\nasm("s_nop // A \\" b");\n')
    assert bench.source_digest(str(a)) == bench.source_digest(str(b))
    assert bench.source_digest(str(a)) != bench.source_digest(str(c))
    assert bench.source_digest(str(a)) != bench.source_digest(str(d))


@pytest.mark.gpu
def test_short_bench_prints_one_contract_line():
    r = subprocess.run([sys.executable, "-u", BENCH, "--steps", "4", "--warmup", "2",
                        "--no-cpu-baseline", "--no-extra", "--no-fused"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    assert TOP_KEYS <= set(d), TOP_KEYS - set(d)
    assert d["n_gpus"] == 1 and d["steps"] == 4 and d["warmup"] == 2
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["workload"] == "decode_llama70b_32k + prefill_causal_8k"
    # Each entry point's object carries its kernel's roofline; the top-level
    # one is the kernel that dominates a step and says so.
    for obj, bound, unit in (("decode", "hbm", "GB/s"), ("prefill", "mfma", "TFLOP/s")):
        rf = d[obj]["roofline"]
        assert ROOFLINE_KEYS <= set(rf), (obj, ROOFLINE_KEYS - set(rf))
        assert rf["bound"] == bound and rf["unit"] == unit
        assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    top = d["roofline"]
    dom = top["dominant_in_step"].split(":")[0]
    assert dom in ("decode", "prefill")
    assert top["kernel"] == d[dom]["roofline"]["kernel"]
    assert top["frac"] == d[dom]["roofline"]["frac"]
    # The decode figure is the back-to-back call rate over the algorithmic bytes.
    dec = d["decode"]
    assert abs(d["value"] - dec["bytes_per_call"] / (dec["us_per_call_back_to_back"] * 1e-6) / 1e9) \
        <= 1e-3 * d["value"]
    assert dec["graph_replay"]["us_per_call"] > 0
