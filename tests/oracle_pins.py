"""Pins that tie the fp64 oracle to things other than itself.

Each ``pin_*`` function takes an oracle namespace ``O`` (the real ``oracle``
package, or a mutant built by ``test_oracle_mutants.py``) and raises
``AssertionError`` when the oracle disagrees with:

* high-precision brute force (mpmath, 50 digits) on tiny shapes, written in the
  plain "sum of exp over sum of exp" form with no max shift;
* a library routine: torch's float64 ``scaled_dot_product_attention`` on the
  CPU (GQA head sharing and an explicit boolean causal mask);
* closed forms: a single key gives ``O = V[0]`` and ``lse = s_0``; identical
  value rows give that row; ``Q = 0`` gives the mean of the visible values and
  ``lse = ln(#visible)``; causal row 0 gives ``V[0]``;
* invariants the pages state or the mathematics fixes: split-KV partials merged
  over any partition and in any order equal one sweep (the merge is
  associative and commutative, ADR-0060@5a76ed4 §4); the per-tile streaming
  update equals one sweep for any tile size (§3 there); jointly permuting
  (key, value) pairs leaves decode unchanged; GQA equals multi-head attention
  with each KV head repeated G times; a causal prefill row equals a decode over
  the keys it sees; huge logits do not overflow;
* for the multi-token decode: brute force per new token, torch's SDPA with an
  explicit mask, and its reductions to plain decode (T_q = 1, and each token
  row over the keys it sees).

Sizes keep the whole file to a few seconds of CPU.
"""

from __future__ import annotations

import math

import numpy as np
import torch

try:
    import mpmath
except ImportError:  # pragma: no cover
    mpmath = None


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, atol=1e-12, rtol=1e-10, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b) - rtol * np.abs(b)) if a.size else 0.0
    assert err <= atol, f"{what}: max excess error {err:.3e}"


# ---------------------------------------------------------------- brute force

def _mp_attention(qrow, keys, vals, scale):
    """High-precision softmax attention of one query row, no max shift."""
    mpmath.mp.dps = 50
    sc = mpmath.mpf(scale)
    w = []
    for krow in keys:
        s = sc * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b))
                             for a, b in zip(qrow, krow))
        w.append(mpmath.e ** s)
    den = mpmath.fsum(w)
    o = [mpmath.fsum(w[j] * mpmath.mpf(float(vals[j][c])) for j in range(len(w))) / den
         for c in range(len(vals[0]))]
    return [float(x) for x in o], float(mpmath.log(den))


def pin_brute_force_decode(O):
    rng = _rng(11)
    for (B, H_q, H_kv, d, lens) in [(1, 2, 1, 4, (5,)), (2, 4, 2, 4, (3, 7)),
                                    (2, 8, 1, 8, (17, 1)), (1, 2, 2, 4, (9,))]:
        cap = max(lens) + 2
        q = rng.standard_normal((B, H_q, d))
        k = rng.standard_normal((B, H_kv, cap, d))
        v = rng.standard_normal((B, H_kv, cap, d))
        scale = 0.7
        o, lse = O.decode(q, k, v, np.array(lens), scale)
        G = H_q // H_kv
        for b in range(B):
            for h in range(H_q):
                kvh = h // G
                L = lens[b]
                ro, rl = _mp_attention(q[b, h], k[b, kvh, :L], v[b, kvh, :L], scale)
                _close(o[b, h], ro, what="brute decode o")
                _close(lse[b, h], rl, what="brute decode lse")


def pin_brute_force_prefill(O):
    rng = _rng(12)
    for (B, H_q, H_kv, d, S_q, S_kv, off, causal) in [
            (1, 2, 1, 4, 5, 5, 0, True), (1, 4, 2, 4, 3, 8, 5, True),
            (2, 2, 1, 4, 4, 6, 0, False), (1, 8, 1, 8, 6, 9, 3, True)]:
        q = rng.standard_normal((B, H_q, S_q, d))
        k = rng.standard_normal((B, H_kv, S_kv, d))
        v = rng.standard_normal((B, H_kv, S_kv, d))
        scale = 0.4
        o, lse = O.prefill(q, k, v, S_kv, scale, causal=causal, causal_offset=off)
        G = H_q // H_kv
        for b in range(B):
            for h in range(H_q):
                for i in range(S_q):
                    top = (off + i + 1) if causal else S_kv
                    ro, rl = _mp_attention(q[b, h, i], k[b, h // G, :top],
                                           v[b, h // G, :top], scale)
                    _close(o[b, h, i], ro, what="brute prefill o")
                    _close(lse[b, h, i], rl, what="brute prefill lse")


# --------------------------------------------------------------- library

def pin_torch_sdpa(O):
    rng = _rng(13)
    for (B, H_q, H_kv, d, S_q, S_kv, off) in [(1, 8, 2, 16, 7, 12, 5),
                                              (2, 4, 4, 8, 10, 10, 0)]:
        q = rng.standard_normal((B, H_q, S_q, d))
        k = rng.standard_normal((B, H_kv, S_kv, d))
        v = rng.standard_normal((B, H_kv, S_kv, d))
        scale = 1.0 / math.sqrt(d)
        for causal in (True, False):
            o, _ = O.prefill(q, k, v, S_kv, scale, causal=causal, causal_offset=off)
            if causal:
                i = torch.arange(S_q)[:, None]
                j = torch.arange(S_kv)[None, :]
                mask = j <= off + i
            else:
                mask = None
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                attn_mask=mask, scale=scale, enable_gqa=True)
            _close(o, ref.numpy(), atol=1e-12, what=f"sdpa causal={causal}")


# ------------------------------------------------------------- closed forms

def pin_single_key(O):
    rng = _rng(14)
    q = rng.standard_normal((2, 8, 16))
    k = rng.standard_normal((2, 2, 4, 16))
    v = rng.standard_normal((2, 2, 4, 16))
    o, lse = O.decode(q, k, v, np.array([1, 1]), 0.3)
    for b in range(2):
        for h in range(8):
            _close(o[b, h], v[b, h // 4, 0], what="single key o")
            _close(lse[b, h], 0.3 * float(np.dot(q[b, h], k[b, h // 4, 0])),
                   what="single key lse")


def pin_identical_values(O):
    rng = _rng(15)
    q = rng.standard_normal((1, 4, 8))
    k = rng.standard_normal((1, 2, 9, 8))
    row = rng.standard_normal(8)
    v = np.broadcast_to(row, (1, 2, 9, 8)).copy()
    o, _ = O.decode(q, k, v, np.array([9]), 1.3)
    for h in range(4):
        _close(o[0, h], row, what="identical V")


def pin_zero_query_mean(O):
    rng = _rng(16)
    B, H_q, H_kv, S_q, S_kv, d, off = 1, 4, 2, 5, 11, 8, 6
    q = np.zeros((B, H_q, S_q, d))
    k = rng.standard_normal((B, H_kv, S_kv, d))
    v = rng.standard_normal((B, H_kv, S_kv, d))
    o, lse = O.prefill(q, k, v, S_kv, 0.5, causal=True, causal_offset=off)
    for h in range(H_q):
        for i in range(S_q):
            n = off + i + 1
            _close(o[0, h, i], v[0, h // 2, :n].mean(axis=0), what="Q=0 mean")
            _close(lse[0, h, i], math.log(n), what="Q=0 lse")
    # scale = 0 on non-zero Q is the same uniform average (decode form).
    q2 = rng.standard_normal((1, H_q, d))
    o2, lse2 = O.decode(q2, k, v, np.array([S_kv]), 0.0)
    for h in range(H_q):
        _close(o2[0, h], v[0, h // 2].mean(axis=0), what="scale=0 mean")
        _close(lse2[0, h], math.log(S_kv), what="scale=0 lse")


def pin_causal_row0(O):
    rng = _rng(17)
    q = rng.standard_normal((1, 4, 6, 8))
    k = rng.standard_normal((1, 1, 6, 8))
    v = rng.standard_normal((1, 1, 6, 8))
    o, _ = O.prefill(q, k, v, 6, 0.9, causal=True, causal_offset=0)
    for h in range(4):
        _close(o[0, h, 0], v[0, 0, 0], what="causal row 0")


def pin_prefill_row_is_decode(O):
    rng = _rng(18)
    B, H_q, H_kv, S_q, S_kv, d, off = 2, 4, 2, 6, 13, 8, 7
    q = rng.standard_normal((B, H_q, S_q, d))
    k = rng.standard_normal((B, H_kv, S_kv, d))
    v = rng.standard_normal((B, H_kv, S_kv, d))
    o, lse = O.prefill(q, k, v, S_kv, 0.6, causal=True, causal_offset=off)
    for i in range(S_q):
        od, ld = O.decode(q[:, :, i], k, v, np.array([off + i + 1] * B), 0.6)
        _close(o[:, :, i], od, what="prefill row == decode")
        _close(lse[:, :, i], ld, what="prefill lse == decode")


def pin_sampled_rows_heads(O):
    rng = _rng(19)
    q = rng.standard_normal((1, 8, 9, 8))
    k = rng.standard_normal((1, 2, 20, 8))
    v = rng.standard_normal((1, 2, 20, 8))
    full, fl = O.prefill(q, k, v, 20, 0.5, causal=True, causal_offset=11)
    rows, heads = np.array([0, 4, 8]), np.array([1, 6])
    sub, sl = O.prefill(q, k, v, 20, 0.5, causal=True, causal_offset=11,
                        rows=rows, heads=heads)
    _close(sub, full[:, heads][:, :, rows], what="sampled rows")
    _close(sl, fl[:, heads][:, :, rows], what="sampled lse")


# ------------------------------------------------------------- invariants

def pin_split_merge_any_partition(O):
    rng = _rng(20)
    d, L = 8, 37
    q = rng.standard_normal((5, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    ref_o, ref_l = O.attend_rows(q, k, v, 0.8, [L] * 5)
    for trial in range(6):
        ncut = int(rng.integers(0, 8))
        cuts = np.sort(rng.choice(np.arange(1, L), size=ncut, replace=False))
        bounds = [0, *cuts.tolist(), L]
        parts = [O.partial(q, k[a:b], v[a:b], 0.8) for a, b in zip(bounds, bounds[1:])]
        if trial % 2:
            parts.append(O.partial(q, k[:0], v[:0], 0.8))    # empty split
        order = rng.permutation(len(parts))
        parts = [parts[i] for i in order]
        while len(parts) > 1:                                # random merge tree
            i = int(rng.integers(0, len(parts) - 1))
            parts[i:i + 2] = [O.merge(parts[i], parts[i + 1])]
        o, lse = O.finalize(parts[0])
        _close(o, ref_o, what="split merge o")
        _close(lse, ref_l, what="split merge lse")


def pin_online_sweep_tiles(O):
    rng = _rng(21)
    d, L = 8, 29
    q = rng.standard_normal((6, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    vis = np.array([1, 5, 16, 17, 28, 29])
    ref_o, ref_l = O.attend_rows(q, k, v, 1.1, vis)
    for tile in (1, 3, 16, L):
        o, lse = O.online_sweep(q, k, v, 1.1, tile, vis)
        _close(o, ref_o, what=f"online sweep tile={tile}")
        _close(lse, ref_l, what=f"online lse tile={tile}")


def pin_permutation_invariance(O):
    rng = _rng(22)
    q = rng.standard_normal((1, 4, 8))
    k = rng.standard_normal((1, 2, 15, 8))
    v = rng.standard_normal((1, 2, 15, 8))
    o, lse = O.decode(q, k, v, np.array([15]), 0.7)
    p = rng.permutation(15)
    o2, lse2 = O.decode(q, k[:, :, p], v[:, :, p], np.array([15]), 0.7)
    _close(o2, o, what="permutation o")
    _close(lse2, lse, what="permutation lse")


def pin_gqa_is_repeated_mha(O):
    rng = _rng(23)
    B, H_q, H_kv, L, d = 2, 8, 2, 10, 8
    q = rng.standard_normal((B, H_q, d))
    k = rng.standard_normal((B, H_kv, L, d))
    v = rng.standard_normal((B, H_kv, L, d))
    o, lse = O.decode(q, k, v, np.array([L, 6]), 0.5)
    G = H_q // H_kv
    kr = np.repeat(k, G, axis=1)
    vr = np.repeat(v, G, axis=1)
    o2, lse2 = O.decode(q, kr, vr, np.array([L, 6]), 0.5)
    _close(o, o2, what="GQA == repeated MHA")
    _close(lse, lse2, what="GQA lse")


def pin_large_logits_and_nan_padding(O):
    rng = _rng(24)
    q = 300.0 * rng.standard_normal((1, 2, 8))
    k = rng.standard_normal((1, 1, 12, 8))
    v = rng.standard_normal((1, 1, 12, 8))
    k[0, 0, 9:] = np.nan           # padding past the valid length
    v[0, 0, 9:] = np.nan
    o, lse = O.decode(q, k, v, np.array([9]), 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "overflow or padding leak"
    for h in range(2):
        s = k[0, 0, :9] @ q[0, h]
        j = int(np.argmax(s))
        gap = np.sort(s)[-1] - np.sort(s)[-2]
        if gap > 50:   # the top key dominates completely
            _close(o[0, h], v[0, 0, j], atol=1e-9, what="argmax row")
        _close(lse[0, h], s.max() + math.log(np.exp(s - s.max()).sum()),
               atol=1e-9, what="large-logit lse")


# ------------------------------------------------------ multi-token decode

def pin_brute_force_decode_multi(O):
    """Each new token, at position L - T_q + t, against high-precision brute
    force over keys 0 .. L - T_q + t."""
    rng = _rng(25)
    for (B, H_q, H_kv, d, T_q, lens) in [(1, 2, 1, 4, 3, (5,)), (2, 4, 2, 4, 2, (2, 7)),
                                         (2, 6, 2, 4, 4, (9, 4))]:
        cap = max(lens) + 3
        q = rng.standard_normal((B, H_q, T_q, d))
        k = rng.standard_normal((B, H_kv, cap, d))
        v = rng.standard_normal((B, H_kv, cap, d))
        o, lse = O.decode_multi(q, k, v, np.array(lens), 0.6)
        G = H_q // H_kv
        for b in range(B):
            for h in range(H_q):
                for t in range(T_q):
                    top = lens[b] - T_q + t + 1
                    ro, rl = _mp_attention(q[b, h, t], k[b, h // G, :top],
                                           v[b, h // G, :top], 0.6)
                    _close(o[b, h, t], ro, what="brute decode_multi o")
                    _close(lse[b, h, t], rl, what="brute decode_multi lse")


def pin_decode_multi_sdpa(O):
    """torch's float64 SDPA with GQA head sharing and an explicit boolean
    mask (new token i of a sequence of length L sees keys j <= L - T_q + i)."""
    rng = _rng(26)
    B, H_q, H_kv, d, T_q = 3, 8, 2, 16, 5
    lens = np.array([5, 12, 31])
    q = rng.standard_normal((B, H_q, T_q, d))
    k = rng.standard_normal((B, H_kv, 32, d))
    v = rng.standard_normal((B, H_kv, 32, d))
    o, _ = O.decode_multi(q, k, v, lens, 0.25)
    for b in range(B):
        L = int(lens[b])
        mask = torch.arange(L)[None, :] <= (L - T_q) + torch.arange(T_q)[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b:b + 1]), torch.from_numpy(k[b:b + 1, :, :L]),
            torch.from_numpy(v[b:b + 1, :, :L]), attn_mask=mask, scale=0.25, enable_gqa=True)
        _close(o[b:b + 1], ref.numpy(), what="decode_multi sdpa")


def pin_decode_multi_special_cases(O):
    """T_q = 1 is plain decode; every token row is a decode over the keys it
    sees; with L = T_q the first token sees only key 0 (O = V[0], lse = s_0)."""
    rng = _rng(27)
    B, H_q, H_kv, d, T_q = 2, 4, 2, 8, 3
    q = rng.standard_normal((B, H_q, T_q, d))
    k = rng.standard_normal((B, H_kv, 10, d))
    v = rng.standard_normal((B, H_kv, 10, d))
    lens = np.array([10, 3])
    o, lse = O.decode_multi(q, k, v, lens, 0.7)
    for t in range(T_q):
        od, ld = O.decode(q[:, :, t], k, v, lens - T_q + t + 1, 0.7)
        _close(o[:, :, t], od, what="decode_multi row == decode")
        _close(lse[:, :, t], ld, what="decode_multi lse == decode")
    o1, l1 = O.decode_multi(q[:, :, :1], k, v, lens, 0.7)
    od, ld = O.decode(q[:, :, 0], k, v, lens, 0.7)
    _close(o1[:, :, 0], od, what="T_q=1 is decode")
    _close(l1[:, :, 0], ld, what="T_q=1 lse")
    for h in range(H_q):
        _close(o[1, h, 0], v[1, h // 2, 0], what="L = T_q first token")
        _close(lse[1, h, 0], 0.7 * float(np.dot(q[1, h, 0], k[1, h // 2, 0])),
               what="L = T_q first token lse")



# ------------------------------------------------------------ chunk stitching

def pin_merge_normalized_chunks(O):
    """Attention over keys split into two chunks at any cut, each chunk's
    normalised (O, LSE) merged, equals attention over all keys (decode) and
    the causal prefill of a chunk after a prefix; merging with an empty side
    (lse = -inf) is the identity; the merge is symmetric."""
    rng = _rng(28)
    d, L = 8, 23
    q = rng.standard_normal((5, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    ref_o, ref_l = O.attend_rows(q, k, v, 0.9, [L] * 5)
    for cut in (1, 7, 22):
        oa, la = O.attend_rows(q, k[:cut], v[:cut], 0.9, [cut] * 5)
        ob, lb = O.attend_rows(q, k[cut:], v[cut:], 0.9, [L - cut] * 5)
        o, lse = O.merge_normalized(oa, la, ob, lb)
        _close(o, ref_o, what=f"stitch cut={cut}")
        _close(lse, ref_l, what=f"stitch lse cut={cut}")
        o2, l2 = O.merge_normalized(ob, lb, oa, la)
        _close(o2, o, what="stitch symmetric")
        _close(l2, lse, what="stitch symmetric lse")
    empty = np.full(5, -np.inf)
    o, lse = O.merge_normalized(ref_o, ref_l, np.full((5, d), np.nan), empty)
    _close(o, ref_o, what="stitch with empty side")
    _close(lse, ref_l, what="stitch with empty side lse")
    # A causal chunk after a cached prefix: the prefix part is unmasked, the
    # chunk's own part is causal; stitched, they are the causal prefill.
    B, H_q, H_kv, S_q, off = 1, 4, 2, 6, 9
    S_kv = off + S_q
    qq = rng.standard_normal((B, H_q, S_q, d))
    kk = rng.standard_normal((B, H_kv, S_kv, d))
    vv = rng.standard_normal((B, H_kv, S_kv, d))
    full_o, full_l = O.prefill(qq, kk, vv, S_kv, 0.5, causal=True, causal_offset=off)
    pre_o, pre_l = O.prefill(qq, kk, vv, off, 0.5, causal=False)
    new_o, new_l = O.prefill(qq, kk[:, :, off:], vv[:, :, off:], S_q, 0.5, causal=True,
                             causal_offset=0)
    o, lse = O.merge_normalized(pre_o, pre_l, new_o, new_l)
    _close(o, full_o, what="prefix + chunk stitch")
    _close(lse, full_l, what="prefix + chunk stitch lse")



# ------------------------------------------------------------- paged caches

def pin_paged_gather_round_trip(O):
    """Scatter contiguous caches into a shuffled page pool (written here with
    explicit loops, pages shared by no one filled with NaN), gather back:
    the valid positions come back unchanged and decode over the pages equals
    decode over the original cache."""
    rng = _rng(29)
    for (B, H_q, H_kv, d, T_q, page, lens) in [(2, 4, 2, 4, 1, 4, (9, 16)),
                                               (3, 8, 2, 4, 3, 2, (3, 7, 12)),
                                               (1, 2, 1, 4, 2, 8, (5,))]:
        top = max(lens)
        k = rng.standard_normal((B, H_kv, top, d))
        v = rng.standard_normal((B, H_kv, top, d))
        q = rng.standard_normal((B, H_q, T_q, d))
        max_pages = (top + page - 1) // page
        num_pages = B * max_pages + 3
        perm = rng.permutation(num_pages)
        table = perm[:B * max_pages].reshape(B, max_pages)
        kp = np.full((num_pages, H_kv, page, d), np.nan)
        vp = np.full((num_pages, H_kv, page, d), np.nan)
        for b in range(B):
            for j in range(lens[b]):
                for h in range(H_kv):
                    kp[table[b, j // page], h, j % page] = k[b, h, j]
                    vp[table[b, j // page], h, j % page] = v[b, h, j]
        kg = O.paged_gather(kp, table, np.array(lens), page)
        for b in range(B):
            assert np.array_equal(kg[b, :, :lens[b]], k[b, :, :lens[b]]), "gather lost a row"
            assert np.all(np.isnan(kg[b, :, lens[b]:])), "gather read past a length"
        o, lse = O.decode_paged(q, kp, vp, table, np.array(lens), page, 0.6)
        ro, rl = O.decode_multi(q, k, v, np.array(lens), 0.6)
        _close(o, ro, what="paged decode")
        _close(lse, rl, what="paged decode lse")



# ------------------------------------------------------------- varlen prefill

def pin_prefill_varlen(O):
    """A ragged batch of causal chunks against brute force per token (token i
    of a chunk of S_q at the end of L positions sees keys 0 .. L - S_q + i);
    an empty chunk is allowed; equal chunk lengths reduce to the multi-token
    decode (whose rows are M-folded head by head, not token-packed); the
    non-causal form sees every key."""
    rng = _rng(30)
    H_q, H_kv, d = 4, 2, 4
    G = H_q // H_kv
    seq = [(3, 7), (0, 4), (5, 5), (1, 9)]          # (S_q, L) per sequence
    cap = 10
    cu = np.concatenate([[0], np.cumsum([sq for sq, _ in seq])])
    q = rng.standard_normal((int(cu[-1]), H_q, d))
    k = rng.standard_normal((len(seq), H_kv, cap, d))
    v = rng.standard_normal((len(seq), H_kv, cap, d))
    lens = np.array([L for _, L in seq])
    o, lse = O.prefill_varlen(q, k, v, cu, lens, 0.8, causal=True)
    for b, (sq, L) in enumerate(seq):
        for i in range(sq):
            for h in range(H_q):
                top = L - sq + i + 1
                ro, rl = _mp_attention(q[cu[b] + i, h], k[b, h // G, :top], v[b, h // G, :top], 0.8)
                _close(o[cu[b] + i, h], ro, what="varlen brute o")
                _close(lse[cu[b] + i, h], rl, what="varlen brute lse")
    onc, _ = O.prefill_varlen(q, k, v, cu, lens, 0.8, causal=False)
    for b, (sq, L) in enumerate(seq):
        for i in range(sq):
            ro, _ = _mp_attention(q[cu[b] + i, 1], k[b, 0, :L], v[b, 0, :L], 0.8)
            _close(onc[cu[b] + i, 1], ro, what="varlen non-causal")
    T_q, lens2 = 3, np.array([3, 8])
    q2 = rng.standard_normal((2, H_q, T_q, d))
    packed = np.transpose(q2, (0, 2, 1, 3)).reshape(2 * T_q, H_q, d)
    o2, l2 = O.prefill_varlen(packed, k[:2], v[:2], np.array([0, 3, 6]), lens2, 0.5)
    om, lm = O.decode_multi(q2, k[:2], v[:2], lens2, 0.5)
    _close(o2, np.transpose(om, (0, 2, 1, 3)).reshape(2 * T_q, H_q, d), what="varlen == multi decode")
    _close(l2, np.transpose(lm, (0, 2, 1)).reshape(2 * T_q, H_q), what="varlen lse == multi decode")
    # A non-causal chunk over an empty cache is the empty result: merged with
    # a real result it leaves that result unchanged.
    oe, le = O.prefill_varlen(q[:3], k[:1], v[:1], np.array([0, 3]), np.array([0]), 0.8,
                              causal=False)
    assert np.all(oe == 0) and np.all(le == -np.inf)
    orl, lrl = O.prefill_varlen(q[:3], k[:1], v[:1], np.array([0, 3]), np.array([6]), 0.8,
                                causal=False)
    om2, lm2 = O.merge_normalized(oe, le, orl, lrl)
    _close(om2, orl, what="empty varlen chunk merges as identity")
    _close(lm2, lrl, what="empty varlen chunk lse")



def pin_prefill_paged(O):
    """Ragged chunks over a shuffled page pool (scattered here with explicit
    loops; unused pages and rows NaN) equal the varlen prefill over the
    contiguous cache they came from, causal and not."""
    rng = _rng(31)
    H_q, H_kv, d, page = 4, 2, 4, 4
    q_lens, lens = (3, 1, 6), (7, 12, 6)
    B, top = len(lens), max(lens)
    cu = np.concatenate([[0], np.cumsum(q_lens)])
    q = rng.standard_normal((int(cu[-1]), H_q, d))
    k = rng.standard_normal((B, H_kv, top, d))
    v = rng.standard_normal((B, H_kv, top, d))
    max_pages = (top + page - 1) // page
    num_pages = B * max_pages + 2
    table = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages)
    kp = np.full((num_pages, H_kv, page, d), np.nan)
    vp = np.full((num_pages, H_kv, page, d), np.nan)
    for b in range(B):
        for j in range(lens[b]):
            for h in range(H_kv):
                kp[table[b, j // page], h, j % page] = k[b, h, j]
                vp[table[b, j // page], h, j % page] = v[b, h, j]
    for causal in (True, False):
        o, lse = O.prefill_paged(q, kp, vp, table, cu, np.array(lens), page, 0.7, causal=causal)
        ro, rl = O.prefill_varlen(q, k, v, cu, np.array(lens), 0.7, causal=causal)
        _close(o, ro, what=f"paged prefill causal={causal}")
        _close(lse, rl, what=f"paged prefill lse causal={causal}")


PINS = [
    pin_brute_force_decode,
    pin_brute_force_prefill,
    pin_torch_sdpa,
    pin_single_key,
    pin_identical_values,
    pin_zero_query_mean,
    pin_causal_row0,
    pin_prefill_row_is_decode,
    pin_sampled_rows_heads,
    pin_split_merge_any_partition,
    pin_online_sweep_tiles,
    pin_permutation_invariance,
    pin_gqa_is_repeated_mha,
    pin_large_logits_and_nan_padding,
    pin_brute_force_decode_multi,
    pin_decode_multi_sdpa,
    pin_decode_multi_special_cases,
    pin_merge_normalized_chunks,
    pin_paged_gather_round_trip,
    pin_prefill_varlen,
    pin_prefill_paged,
]
