"""fp64 reference for grouped-query attention (decode and causal prefill).

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is computed.  The pages state that the kernel is FlashAttention tiling
with an online softmax and a fused P.V, FlashDecoding's split-KV with a
log-sum-exp merge, and Ring Attention's rotated KV blocks folded by the same
online softmax, and that no new mathematics is introduced (ADR-0060@5a76ed4,
"Status", the "Algorithm lineage" paragraph).  All three reach plain softmax
attention exactly (up to rounding order), so the reference result is that
definition written out: ``attend_rows`` below.

The remaining functions restate the page's algorithm steps in the pages'
order and notation -- the split partial ``(m, l, O)``, the merge, the final
normalisation and the per-tile streaming update -- so that tests can check,
in fp64, that composing them gives the definition for any partition and any
tile size.

Readings taken where the pages are silent:
  * query head ``h`` reads KV head ``h // G`` (the G query rows of one KV head
    are stacked contiguously, ADR-0060@5a76ed4 §0 "CUBE Group" and §0.5.3
    INPUTS, where Q is ``[G, T_q, d]`` per KV head);
  * the causal mask is the visibility set ``j <= causal_offset + i`` rather
    than an additive constant (the pages say "additive causal mask" without a
    value, ADR-0060@5a76ed4 §3 and §5.4);
  * ``scale`` is applied to ``q . k`` before masking and the max (§3 there);
  * the natural-log LSE ``m + ln(l)`` is the exported statistic.

All arithmetic is numpy float64.  Inputs of any float dtype are upcast to
float64 first; callers pass the bf16-rounded values the GPU sees.
"""

from __future__ import annotations

import numpy as np


def kv_head_of(h: int, H_q: int, H_kv: int) -> int:
    """KV head read by query head ``h``: ``h // G`` with ``G = H_q / H_kv``.

    ADR-0060@5a76ed4 §0 "Reference dimensions" (G = H_q / H_kv) and the
    "CUBE Group" paragraph (the G query heads of one KV head are M-folded,
    ``[G, T_q, d] -> [G*T_q, d]``).
    """
    if H_q % H_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    return h // (H_q // H_kv)


def attend_rows(q_rows, k, v, scale: float, visible_len):
    """The definition: ``softmax(scale * q k^T over visible keys) v`` in fp64.

    q_rows: ``[n, d]`` query rows of one query head (or of the G heads that
    share one KV head).
    k, v:   ``[L, d]`` keys and values of the KV head (row j = position j).
    visible_len: ``[n]`` ints; row i sees keys ``0 .. visible_len[i]-1``.
        Every entry must be >= 1 and <= L.

    Returns ``(o [n, d], lse [n])`` with ``lse = max_s + ln(sum exp(s - max_s))``
    over the visible keys.  Rows are independent; they are evaluated together
    as matrix products.  Keys past the largest visible length are not read,
    so NaN padding there cannot leak in.
    """
    q = np.asarray(q_rows, dtype=np.float64)
    vl = np.asarray(visible_len, dtype=np.int64).reshape(-1)
    n = q.shape[0]
    if vl.shape[0] != n:
        raise ValueError("visible_len must have one entry per query row")
    if n and (vl.min() < 1 or vl.max() > k.shape[0]):
        raise ValueError("visible lengths must lie in [1, L]")
    top = int(vl.max()) if n else 0
    k = np.asarray(k[:top], dtype=np.float64)
    v = np.asarray(v[:top], dtype=np.float64)
    s = float(scale) * (q @ k.T)                       # [n, top]
    visible = np.arange(top)[None, :] < vl[:, None]
    s = np.where(visible, s, -np.inf)
    mx = s.max(axis=1)
    w = np.exp(s - mx[:, None])                        # hidden keys get 0
    den = w.sum(axis=1)
    o = (w @ v) / den[:, None]
    lse = mx + np.log(den)
    return o, lse


def decode(q, k_cache, v_cache, kv_lens, scale: float):
    """Decode attention (T_q = 1): every query attends to all valid keys.

    q: ``[B, H_q, d]``; k_cache, v_cache: ``[B, H_kv, kv_cap, d]``;
    kv_lens: ``[B]`` valid lengths (keys ``0 .. kv_lens[b]-1``).
    Decode is unmasked: the one new query attends to all past KV
    (ADR-0060@5a76ed4 §5.2).  The G query heads of a KV head are evaluated
    together against it.  Returns ``(o [B, H_q, d], lse [B, H_q])``.
    """
    q = np.asarray(q)
    B, H_q, d = q.shape
    H_kv = k_cache.shape[1]
    lens = np.asarray(kv_lens, dtype=np.int64).reshape(-1)
    o = np.empty((B, H_q, d), dtype=np.float64)
    lse = np.empty((B, H_q), dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        for kv in range(H_kv):
            heads = [h for h in range(H_q) if kv_head_of(h, H_q, H_kv) == kv]
            ob, lb = attend_rows(q[b, heads], k_cache[b, kv, :L], v_cache[b, kv, :L],
                                 scale, [L] * len(heads))
            o[b, heads] = ob
            lse[b, heads] = lb
    return o, lse


def decode_multi_visible_len(L: int, G: int, T_q: int):
    """Visible key count of each M-folded row of a multi-token decode.

    The ``T_q`` new tokens of a sequence of ``L`` valid positions are its last
    ``T_q`` positions (their K/V rows are already in the cache, precondition
    P3 of ADR-0060@5a76ed4 §0.5.1), so the query block starts at
    ``q_start = L - T_q`` (``q_block_meta``, §0.5.3) and token ``t`` sees keys
    ``j <= q_start + t``.  The G query heads are stacked head by head,
    ``[G, T_q] -> [G*T_q]`` (§3 running state, §5.2): row ``r`` is token
    ``r % T_q`` of head ``r // T_q``.
    """
    t = np.tile(np.arange(T_q, dtype=np.int64), G)
    return (L - T_q) + t + 1


def decode_multi(q, k_cache, v_cache, kv_lens, scale: float):
    """Decode of ``T_q`` new tokens per sequence (multi-token / speculative
    decode): the G heads x T_q tokens of one KV head are M-folded into
    ``G*T_q`` rows that share every K/V tile (ADR-0060@5a76ed4 §3, §5.2),
    with the causal tail of ``decode_multi_visible_len``.

    q: ``[B, H_q, T_q, d]``; k_cache, v_cache: ``[B, H_kv, kv_cap, d]``;
    kv_lens: ``[B]`` valid lengths, each ``>= T_q``.
    Returns ``(o [B, H_q, T_q, d], lse [B, H_q, T_q])``.
    """
    q = np.asarray(q)
    B, H_q, T_q, d = q.shape
    H_kv = k_cache.shape[1]
    G = H_q // H_kv
    lens = np.asarray(kv_lens, dtype=np.int64).reshape(-1)
    o = np.empty((B, H_q, T_q, d), dtype=np.float64)
    lse = np.empty((B, H_q, T_q), dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        if L < T_q:
            raise ValueError("every sequence must hold its T_q new tokens")
        vl = decode_multi_visible_len(L, G, T_q)
        for kv in range(H_kv):
            heads = [h for h in range(H_q) if kv_head_of(h, H_q, H_kv) == kv]
            rows = q[b, heads].reshape(G * T_q, d)            # M-fold [G, T_q, d] -> [G*T_q, d]
            ob, lb = attend_rows(rows, k_cache[b, kv, :L], v_cache[b, kv, :L], scale, vl)
            o[b, heads] = ob.reshape(G, T_q, d)
            lse[b, heads] = lb.reshape(G, T_q)
    return o, lse


def prefill_varlen(q, k, v, cu_seqlens_q, kv_lens, scale: float, causal: bool = True):
    """A batch of prefill chunks of different lengths (token-packed).

    q: ``[total_q, H_q, d]`` with sequence ``b``'s chunk at rows
    ``cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1``; k, v: ``[B, H_kv, kv_cap, d]``
    with ``kv_lens[b]`` valid positions.  Each chunk is the last ``S_q_b``
    positions of its sequence (its K/V already in the cache, precondition P3
    of ADR-0060@5a76ed4 §0.5.1), so with a causal mask its token ``i`` sees
    keys ``j <= kv_lens[b] - S_q_b + i`` -- ``prefill`` with
    ``causal_offset = kv_lens[b] - S_q_b`` (``q_block_meta``, §0.5.3); without
    one, all ``kv_lens[b]`` keys.  A non-causal chunk whose sequence has no
    cached key at all has no visible key in any row: O = 0 and lse = -inf,
    the empty result of ``merge_normalized`` (it leaves the other side
    unchanged).  Returns ``(o [total_q, H_q, d], lse [total_q, H_q])``.
    """
    q = np.asarray(q)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64).reshape(-1)
    lens = np.asarray(kv_lens, dtype=np.int64).reshape(-1)
    total, H_q, d = q.shape
    o = np.empty((total, H_q, d), dtype=np.float64)
    lse = np.empty((total, H_q), dtype=np.float64)
    for b in range(len(cu) - 1):
        t0, t1, L = int(cu[b]), int(cu[b + 1]), int(lens[b])
        S_q = t1 - t0
        if S_q == 0:
            continue
        if causal and S_q > L:
            raise ValueError("a causal chunk must be the last S_q of its sequence's positions")
        if L == 0:
            o[t0:t1] = 0.0
            lse[t0:t1] = -np.inf
            continue
        qb = np.transpose(q[t0:t1], (1, 0, 2))[None]            # [1, H_q, S_q, d]
        ob, lb = prefill(qb, k[b:b + 1], v[b:b + 1], L, scale, causal=causal,
                         causal_offset=L - S_q)
        o[t0:t1] = np.transpose(ob[0], (1, 0, 2))
        lse[t0:t1] = lb[0].T
    return o, lse


def paged_gather(pages, block_table, kv_lens, page_size: int):
    """A paged cache laid out contiguously: sequence ``b``'s position ``j``
    lives in physical page ``block_table[b, j // page_size]`` at row
    ``j % page_size``.

    pages: ``[num_pages, H_kv, page_size, d]``; block_table: ``[B, max_pages]``.
    Returns ``[B, H_kv, max(kv_lens), d]`` float64 with positions past a
    sequence's length set to NaN (they must never be read).
    """
    pages = np.asarray(pages, dtype=np.float64)
    table = np.asarray(block_table, dtype=np.int64)
    lens = np.asarray(kv_lens, dtype=np.int64).reshape(-1)
    B, H_kv, d = table.shape[0], pages.shape[1], pages.shape[3]
    top = int(lens.max())
    out = np.full((B, H_kv, top, d), np.nan)
    for b in range(B):
        for j in range(int(lens[b])):
            out[b, :, j] = pages[table[b, j // page_size], :, j % page_size]
    return out


def decode_paged(q, k_pages, v_pages, block_table, kv_lens, page_size: int, scale: float):
    """Decode of ``T_q >= 1`` new tokens per sequence (as ``decode_multi``)
    over a paged K/V cache: the attention is unchanged, only the cache
    layout differs (``paged_gather``).  q: ``[B, H_q, T_q, d]``."""
    k = paged_gather(k_pages, block_table, kv_lens, page_size)
    v = paged_gather(v_pages, block_table, kv_lens, page_size)
    return decode_multi(q, k, v, kv_lens, scale)


def prefill_paged(q, k_pages, v_pages, block_table, cu_seqlens_q, kv_lens, page_size: int,
                  scale: float, causal: bool = True):
    """Varlen prefill (``prefill_varlen``) over a paged K/V cache: the
    attention is unchanged, only the cache layout differs (``paged_gather``).
    q: ``[total_q, H_q, d]`` token-packed."""
    k = paged_gather(k_pages, block_table, kv_lens, page_size)
    v = paged_gather(v_pages, block_table, kv_lens, page_size)
    return prefill_varlen(q, k, v, cu_seqlens_q, kv_lens, scale, causal=causal)


def prefill_visible_len(rows, S_kv: int, causal: bool, causal_offset: int):
    """Visible key count per query row of a prefill chunk.

    With a causal mask, query ``i`` of a chunk appended after
    ``causal_offset`` cached tokens sees keys ``j <= causal_offset + i``
    (ADR-0060@5a76ed4 §0.5.3 ``q_block_meta {q_start, T_q}`` and §5.4: tiles
    wholly after the query block are invisible).  Without it, all ``S_kv``.
    """
    rows = np.asarray(rows, dtype=np.int64)
    if causal:
        return causal_offset + rows + 1
    return np.full(rows.shape, S_kv, dtype=np.int64)


def prefill(q, k, v, S_kv: int, scale: float, causal: bool = True,
            causal_offset: int = 0, rows=None, heads=None):
    """Prefill attention over a chunk of ``S_q`` queries.

    q: ``[B, H_q, S_q, d]``; k, v: ``[B, H_kv, kv_cap, d]`` (first ``S_kv``
    positions valid).  ``rows`` selects query positions (default: all) and
    ``heads`` query heads (default: all), for sampled checks of large cases.
    Returns ``(o [B, len(heads), len(rows), d], lse [B, len(heads), len(rows)])``.
    """
    q = np.asarray(q)
    B, H_q, S_q, d = q.shape
    H_kv = k.shape[1]
    rows = np.arange(S_q) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(H_q) if heads is None else np.asarray(heads, dtype=np.int64)
    vl = prefill_visible_len(rows, S_kv, causal, causal_offset)
    o = np.empty((B, len(heads), len(rows), d), dtype=np.float64)
    lse = np.empty((B, len(heads), len(rows)), dtype=np.float64)
    top = int(vl.max()) if len(rows) else 0
    for b in range(B):
        for hi, h in enumerate(heads):
            kv = kv_head_of(int(h), H_q, H_kv)
            kk = np.asarray(k[b, kv, :top], dtype=np.float64)
            vv = np.asarray(v[b, kv, :top], dtype=np.float64)
            for r0 in range(0, len(rows), 256):       # bounded [rows, keys] block
                r1 = min(r0 + 256, len(rows))
                ob, lb = attend_rows(q[b, h][rows[r0:r1]], kk, vv, scale, vl[r0:r1])
                o[b, hi, r0:r1] = ob
                lse[b, hi, r0:r1] = lb
    return o, lse


# ---------------------------------------------------------------------------
# The pages' algorithm, step by step (fp64).  Used by tests to confirm that
# split-KV partials merged in any order, and the per-tile streaming update at
# any tile size, reach the definition above.
# ---------------------------------------------------------------------------

def partial(q_rows, k, v, scale: float):
    """Unnormalised split partial ``(m, l, O)`` over one contiguous KV split.

    After its sweep each split holds ``m = max_j s_j``,
    ``l = sum_j exp(s_j - m)`` and ``O = sum_j exp(s_j - m) v_j``, not yet
    divided by ``l`` (ADR-0060@5a76ed4 §4 "Reduction"; ADR-001@1897945
    §0.5.4, the intermediate partial table).  ``k``/``v`` hold the split's
    keys; an empty split returns the identity ``(-inf, 0, 0)``.
    """
    q = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape[0], v.shape[1]
    if k.shape[0] == 0:
        return (np.full(n, -np.inf), np.zeros(n), np.zeros((n, d)))
    s = float(scale) * (q @ k.T)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return m, p.sum(axis=1), p @ v


def merge(a, b):
    """Log-sum-exp merge of two partials (ADR-0060@5a76ed4 §4 ``merge``).

    ``m = max(m_a, m_b)``; each side is weighted by ``exp(m_side - m)``;
    ``l`` and ``O`` are the weighted sums.  A side with ``m = -inf`` (an
    empty split) gets weight 0, so ``(-inf, 0, 0)`` is the identity.
    """
    m_a, l_a, o_a = a
    m_b, l_b, o_b = b
    m = np.maximum(m_a, m_b)
    with np.errstate(invalid="ignore"):
        sa = np.where(np.isneginf(m_a), 0.0, np.exp(m_a - m))
        sb = np.where(np.isneginf(m_b), 0.0, np.exp(m_b - m))
    return m, l_a * sa + l_b * sb, o_a * sa[:, None] + o_b * sb[:, None]


def merge_normalized(o_a, lse_a, o_b, lse_b):
    """Stitch two attention results over disjoint key sets of the same query
    rows, each given normalised with its LSE (chunk stitching).

    A normalised result is the partial ``(m, l, O) = (lse, 1, O)``: its
    weights relative to ``lse`` sum to one.  So the merge of ADR-0060@5a76ed4
    §4 applies unchanged, followed by the one normalisation (``finalize``).
    o_*: ``[..., d]``; lse_*: ``[...]`` natural log.  A side with
    ``lse = -inf`` (no visible key) contributes nothing.
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    shape, d = lse_a.shape, o_a.shape[-1]
    def as_partial(o, lse):
        lse = lse.reshape(-1)
        # An empty side gets weight 0 in the merge; its O (undefined) is zeroed
        # so that 0 * NaN cannot reach the sum.
        o = np.where(np.isneginf(lse)[:, None], 0.0, o.reshape(-1, d))
        return lse, np.ones(lse.size), o

    o, lse = finalize(merge(as_partial(o_a, lse_a), as_partial(o_b, lse_b)))
    return o.reshape(*shape, d), lse.reshape(shape)


def finalize(t):
    """Normalise once at the end: ``O / l`` and ``lse = m + ln(l)``
    (ADR-0060@5a76ed4 §4, "normalise once" after the merge)."""
    m, l, o = t
    return o / l[:, None], m + np.log(l)


def online_sweep(q_rows, k, v, scale: float, tile: int, visible_len=None):
    """The per-tile streaming update over tiles of ``tile`` keys.

    Running state starts at ``(m, l, O) = (-inf, 0, 0)``.  For each tile:
    ``S = scale * q K_j^T`` (masked entries removed), ``m_new = max(m,
    rowmax S)``, ``P = exp(S - m_new)``, ``corr = exp(m - m_new)``,
    ``l = l*corr + rowsum P``, ``O = O*corr + P V_j``, ``m = m_new``
    (ADR-0060@5a76ed4 §3 "Per-tile op sequence").  A tile holding no visible
    key for a row leaves that row untouched, as a wholly-future tile is
    skipped (§5.4 there).  Returns the normalised ``(o, lse)``.
    """
    q = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, L, d = q.shape[0], k.shape[0], v.shape[1]
    vl = (np.full(n, L) if visible_len is None
          else np.asarray(visible_len, dtype=np.int64).reshape(-1))
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    o = np.zeros((n, d))
    for j0 in range(0, L, tile):
        j1 = min(j0 + tile, L)
        s = float(scale) * (q @ k[j0:j1].T)
        vis = np.arange(j0, j1)[None, :] < vl[:, None]
        s = np.where(vis, s, -np.inf)
        live = vis.any(axis=1)
        m_new = np.where(live, np.maximum(m, s.max(axis=1)), m)
        with np.errstate(invalid="ignore"):
            p = np.where(vis, np.exp(s - m_new[:, None]), 0.0)
            # exp(-inf - finite) = 0 discards the empty initial state.
            corr = np.where(live, np.exp(m - m_new), 1.0)
        l = l * corr + p.sum(axis=1)
        o = o * corr[:, None] + p @ v[j0:j1]
        m = m_new
    return o / l[:, None], m + np.log(l)
