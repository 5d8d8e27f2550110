"""Workload shapes against the dimensions the pages print (CPU only)."""

import json
import math
import os

import numpy as np

from gqa_flashattention_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "llama3_70b_attention_dims.json")


def test_llama_geometry_matches_pages():
    g = json.load(open(GOLDEN))
    assert g["G"] == g["H_q"] // g["H_kv"]
    for w in inputs.WORKLOADS.values():
        if w.name == "decode_small_f32":
            assert (w.H_q, w.H_kv, w.d) == (g["G"], 1, g["d"])   # one KV group
            continue
        assert (w.H_q, w.H_kv, w.d, w.G) == (g["H_q"], g["H_kv"], g["d"], g["G"])
        assert w.scale == np.float32(1.0 / math.sqrt(g["d"]))


def test_algorithmic_work_counts():
    w2 = inputs.WORKLOADS["decode_llama70b_32k"]
    assert w2.kv_bytes() == 134217728            # 128 MiB of K+V
    assert w2.decode_bytes() == 134250496
    w3 = inputs.WORKLOADS["decode_ragged_b4"]
    assert w3.decode_bytes() == 973209600
    w4 = inputs.WORKLOADS["prefill_causal_8k"]
    assert w4.visible_pairs_per_head() == 8192 * 8193 // 2
    assert w4.prefill_flops() == 4 * 128 * 64 * 33558528
    w5 = inputs.WORKLOADS["prefill_chunk_64k"]
    assert w5.visible_pairs_per_head() == 503320576


def test_generator_is_seeded_and_nan_padded():
    w = inputs.Workload("t", "decode", B=2, H_q=4, H_kv=2, d=8, dtype="bf16",
                        lens=(3, 5), kv_cap=6)
    a = inputs.make_decode(w, seed=5)
    b = inputs.make_decode(w, seed=5)
    for key in ("q", "k", "v"):
        assert a[key].equal(b[key]) or (a[key].isnan() == b[key].isnan()).all()
    assert a["k"][0, :, 3:].isnan().all() and not a["k"][0, :, :3].isnan().any()
    assert a["v"][1, :, 5:].isnan().all() and not a["v"][1, :, :5].isnan().any()
    rows = inputs.sample_rows(8192, 512, seed=3)
    assert len(rows) == 512 and len(set(rows)) == 512
    assert {0, 1, 63, 64, 127, 128, 8191} <= set(rows)
