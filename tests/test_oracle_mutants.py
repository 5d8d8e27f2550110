"""Plant plausible mistakes in a copy of the oracle and check a pin catches each.

Each mutant is the oracle's source with one textual change (a dropped term, a
wrong sign, a wrong index or operand), executed as a fresh module on the CPU.
The pins must reject every mutant: otherwise they would not pin the oracle.
"""

import os
import types

import pytest

import oracle_pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "attention.py")

MUTANTS = {
    "head_map_modulo": ("return h // (H_q // H_kv)", "return h % H_kv"),
    "dropped_scale": ("s = float(scale) * (q @ k.T)                       # [n, top]",
                      "s = (q @ k.T)"),
    "causal_off_by_one": ("return causal_offset + rows + 1", "return causal_offset + rows + 2"),
    "max_sign": ("w = np.exp(s - mx[:, None])", "w = np.exp(s + mx[:, None])"),
    "lse_dropped_max": ("lse = mx + np.log(den)\n    return o, lse", "lse = np.log(den)\n    return o, lse"),
    "values_from_keys": ("o = (w @ v) / den[:, None]", "o = (w @ k) / den[:, None]"),
    "mask_off_by_one": ("visible = np.arange(top)[None, :] < vl[:, None]",
                        "visible = np.arange(top)[None, :] <= vl[:, None]"),
    "merge_weight_sign": ("sa = np.where(np.isneginf(m_a), 0.0, np.exp(m_a - m))",
                          "sa = np.where(np.isneginf(m_a), 0.0, np.exp(m - m_a))"),
    "sweep_no_rescale": ("o = o * corr[:, None] + p @ v[j0:j1]", "o = o + p @ v[j0:j1]"),
    "partial_unshifted": ("p = np.exp(s - m[:, None])", "p = np.exp(s)"),
    "decode_drops_last_key": ("v_cache[b, kv, :L],\n", "v_cache[b, kv, 1:L + 1],\n"),
    "keys_reversed": ("s = float(scale) * (q @ k.T)", "s = float(scale) * (q @ k[::-1].T)"),
    "multi_tail_short": ("return (L - T_q) + t + 1", "return (L - T_q) + t"),
    "multi_fold_token_major": ("rows = q[b, heads].reshape(G * T_q, d)",
                               "rows = q[b, heads].transpose(1, 0, 2).reshape(G * T_q, d)"),
    "multi_tokens_repeated": ("t = np.tile(np.arange(T_q, dtype=np.int64), G)",
                              "t = np.repeat(np.arange(T_q, dtype=np.int64), G)"),
    "stitch_empty_o_kept": ("o = np.where(np.isneginf(lse)[:, None], 0.0, o.reshape(-1, d))",
                            "o = o.reshape(-1, d)"),
    "stitch_weights_swapped": ("o, lse = finalize(merge(as_partial(o_a, lse_a), as_partial(o_b, lse_b)))",
                               "o, lse = finalize(merge(as_partial(o_a, lse_b), as_partial(o_b, lse_a)))"),
    "paged_row_shift": ("out[b, :, j] = pages[table[b, j // page_size], :, j % page_size]",
                        "out[b, :, j] = pages[table[b, j // page_size], :, (j + 1) % page_size]"),
    "paged_wrong_page": ("out[b, :, j] = pages[table[b, j // page_size], :, j % page_size]",
                         "out[b, :, j] = pages[table[b, j % page_size], :, j % page_size]"),
    "varlen_offset_zero": ("causal_offset=L - S_q)\n        o[t0:t1]", "causal_offset=0)\n        o[t0:t1]"),
    "varlen_heads_tokens_swapped": ("qb = np.transpose(q[t0:t1], (1, 0, 2))[None]",
                                    "qb = q[t0:t1].reshape(q.shape[1], t1 - t0, q.shape[2])[None]"),
    "visible_ignored": ("vis = np.arange(j0, j1)[None, :] < vl[:, None]",
                        "vis = np.arange(j0, j1)[None, :] < L + 0 * vl[:, None]"),
}


def _load_mutant(old, new):
    src = open(SRC_PATH).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name):
    if oracle_pins.mpmath is None:
        pytest.skip("mpmath not importable")
    mutant = _load_mutant(*MUTANTS[name])
    caught = []
    for pin in oracle_pins.PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError, IndexError, FloatingPointError) as e:
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin rejects mutant {name}"
