"""Seeded synthetic inputs shared by the tests, the bench and the oracle leg.

This module holds workload shapes and random number generation only: none of
the attention arithmetic.  It imports nothing from ``oracle/`` or from the
HIP binding, so both sides of a parity check can take their inputs from it.

Recipe.  Every tensor is i.i.d. N(0, 1) drawn in float32 from a
``torch.Generator`` seeded with ``seed * 16 + tensor_id`` on the device the
tensor lives on, then rounded to bfloat16 (round-to-nearest-even, torch's
cast) for the bf16 workloads.  Cache positions past a sequence's valid length
are filled with NaN, so a kernel that reads padding poisons its output.  The
softmax scale is the float32 value of ``1/sqrt(d)``.

Workloads follow the Llama3-70B attention geometry of the pages (H_q = 64,
H_kv = 8, G = 8, d = 128; ADR-0060@5a76ed4 §0 "Reference dimensions") at the
lengths of the five measured cases below.  No dataset or trained weights are
involved.
"""

from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "decode", "decode_multi" or "prefill"
    B: int
    H_q: int
    H_kv: int
    d: int
    dtype: str           # "f32" or "bf16"
    lens: tuple = ()     # decode: valid KV length per sequence
    kv_cap: int = 0      # decode: cache capacity (padded length)
    S_q: int = 0         # prefill: query chunk length
    S_kv: int = 0        # prefill: keys in the cache
    causal: bool = True
    offset: int = 0      # prefill: cached tokens before the chunk
    T_q: int = 1         # decode_multi: new tokens per sequence (the last T_q positions)
    page_size: int = 0   # decode_paged: positions per page of the paged cache
    q_lens: tuple = ()   # prefill_varlen: chunk length per sequence (lens: its cache length)

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def max_kv_len(self) -> int:
        if self.kind.startswith("decode") or self.kind in ("prefill_varlen", "prefill_paged"):
            return max(self.lens)
        return self.S_kv

    def kv_bytes(self) -> int:
        """K+V bytes a decode step must read: valid keys only, padding excluded."""
        return 2 * sum(self.lens) * self.H_kv * self.d * self.elem_bytes

    def decode_bytes(self) -> int:
        """Algorithmic bytes of one decode call: K+V of the valid keys, Q and O
        (T_q rows per head for the multi-token decode)."""
        qo = 2 * self.B * self.H_q * self.T_q * self.d * self.elem_bytes
        return self.kv_bytes() + qo

    def decode_multi_flops(self) -> int:
        """Algorithmic FLOPs of a multi-token decode: 4*d per visible
        (token, key) pair and query head; token t of a sequence of length L
        sees L - T_q + t + 1 keys."""
        pairs = sum(self.T_q * (L - self.T_q) + self.T_q * (self.T_q + 1) // 2 for L in self.lens)
        return 4 * self.d * self.H_q * pairs

    def visible_pairs_per_head(self) -> int:
        """(query, key) pairs a causal prefill chunk must score, per head."""
        if not self.causal:
            return self.S_q * self.S_kv
        return sum(self.offset + i + 1 for i in range(self.S_q))

    def prefill_flops(self) -> int:
        """Algorithmic FLOPs: 2*d for Q.K^T plus 2*d for P.V per visible pair."""
        if self.kind in ("prefill_varlen", "prefill_paged"):
            return 4 * self.d * self.H_q * self.varlen_visible_pairs()
        return 4 * self.d * self.B * self.H_q * self.visible_pairs_per_head()

    def varlen_visible_pairs(self) -> int:
        """(query, key) pairs per head of a varlen batch: chunk b (S_q tokens,
        the newest of L positions) scores L - S_q + i + 1 keys for token i
        when causal, L otherwise."""
        if not self.causal:
            return sum(sq * L for sq, L in zip(self.q_lens, self.lens))
        return sum(sq * (L - sq) + sq * (sq + 1) // 2 for sq, L in zip(self.q_lens, self.lens))

    @property
    def total_q(self) -> int:
        return sum(self.q_lens)


WORKLOADS = {
    "decode_small_f32": Workload("decode_small_f32", "decode", B=1, H_q=8, H_kv=1,
                                 d=128, dtype="f32", lens=(256,), kv_cap=256),
    "decode_llama70b_32k": Workload("decode_llama70b_32k", "decode", B=1, H_q=64,
                                    H_kv=8, d=128, dtype="bf16", lens=(32768,),
                                    kv_cap=32768),
    "decode_ragged_b4": Workload("decode_ragged_b4", "decode", B=4, H_q=64, H_kv=8,
                                 d=128, dtype="bf16",
                                 lens=(8192, 32768, 65536, 131072), kv_cap=131072),
    "prefill_causal_8k": Workload("prefill_causal_8k", "prefill", B=1, H_q=64,
                                  H_kv=8, d=128, dtype="bf16", S_q=8192,
                                  S_kv=8192, causal=True, offset=0),
    "prefill_chunk_64k": Workload("prefill_chunk_64k", "prefill", B=1, H_q=64,
                                  H_kv=8, d=128, dtype="bf16", S_q=8192,
                                  S_kv=65536, causal=True, offset=57344),
    # Multi-token (speculative) decode on the 32K-key cache: 4 and 16 new
    # tokens per sequence, G*T_q = 32 and 128 folded rows (and 2, below).
    "decode_multi_llama70b_32k_t4": Workload("decode_multi_llama70b_32k_t4", "decode_multi",
                                             B=1, H_q=64, H_kv=8, d=128, dtype="bf16",
                                             lens=(32768,), kv_cap=32768, T_q=4),
    "decode_multi_llama70b_32k_t16": Workload("decode_multi_llama70b_32k_t16", "decode_multi",
                                              B=1, H_q=64, H_kv=8, d=128, dtype="bf16",
                                              lens=(32768,), kv_cap=32768, T_q=16),
    # T_q = 2 (one draft token): G*T_q = 16 rows, the decode kernel's tile.
    "decode_multi_llama70b_32k_t2": Workload("decode_multi_llama70b_32k_t2", "decode_multi",
                                             B=1, H_q=64, H_kv=8, d=128, dtype="bf16",
                                             lens=(32768,), kv_cap=32768, T_q=2),
    # The decode_llama70b_32k cache in a pool of 64-position pages placed in
    # a seeded random order (T_q = 1).
    "decode_paged_llama70b_32k_p64": Workload("decode_paged_llama70b_32k_p64", "decode_paged",
                                              B=1, H_q=64, H_kv=8, d=128, dtype="bf16",
                                              lens=(32768,), kv_cap=32768, T_q=1, page_size=64),
    # A chunked-prefill batch (continuous batching): eight sequences, each
    # appending a chunk of a different length (a full 8K prompt, a long
    # chunk over a 64K context, mid-size chunks, a ragged 37-token tail and
    # a single decode-like token) to its own cache; 16166 query tokens.
    "prefill_varlen_llama70b_b8": Workload("prefill_varlen_llama70b_b8", "prefill_varlen",
                                           B=8, H_q=64, H_kv=8, d=128, dtype="bf16",
                                           q_lens=(8192, 4096, 2048, 1024, 512, 256, 37, 1),
                                           lens=(8192, 12288, 32768, 2048, 65536, 4096, 300,
                                                 16384),
                                           kv_cap=65536, causal=True),
    # The same batch with its caches in a pool of 16-position pages placed
    # in a seeded random order.
    "prefill_paged_llama70b_b8_p16": Workload("prefill_paged_llama70b_b8_p16", "prefill_paged",
                                              B=8, H_q=64, H_kv=8, d=128, dtype="bf16",
                                              q_lens=(8192, 4096, 2048, 1024, 512, 256, 37, 1),
                                              lens=(8192, 12288, 32768, 2048, 65536, 4096, 300,
                                                    16384),
                                              kv_cap=65536, causal=True, page_size=16),
}

# Seed per workload: 20260000 + its position in the list above (1-based).
SEEDS = {name: 20260000 + i + 1 for i, name in enumerate(WORKLOADS)}


def _gen(device, seed: int, tensor_id: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 16 + tensor_id)
    return g


def randn(shape, dtype, device, seed: int, tensor_id: int) -> torch.Tensor:
    """N(0,1) in float32 from a seeded generator, then cast to ``dtype``."""
    g = _gen(device, seed, tensor_id)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)


def make_decode(w: Workload, device="cpu", seed=None, nan_pad=True, lens=None):
    """Decode inputs: q ``[B,H_q,d]``, k/v ``[B,H_kv,kv_cap,d]``, kv_lens int32."""
    seed = SEEDS.get(w.name, 1) if seed is None else seed
    lens = tuple(w.lens) if lens is None else tuple(lens)
    dt = w.torch_dtype
    q = randn((w.B, w.H_q, w.d), dt, device, seed, 0)
    k = randn((w.B, w.H_kv, w.kv_cap, w.d), dt, device, seed, 1)
    v = randn((w.B, w.H_kv, w.kv_cap, w.d), dt, device, seed, 2)
    if nan_pad:
        for b, L in enumerate(lens):
            if L < w.kv_cap:
                k[b, :, L:].fill_(float("nan"))
                v[b, :, L:].fill_(float("nan"))
    kv_lens = torch.tensor(lens, dtype=torch.int32, device=device)
    return {"q": q, "k": k, "v": v, "kv_lens": kv_lens}


def make_decode_multi(w: Workload, device="cpu", seed=None, nan_pad=True, lens=None):
    """Multi-token decode inputs: q ``[B,H_q,T_q,d]``, k/v ``[B,H_kv,kv_cap,d]``
    (the new tokens' rows included), kv_lens int32."""
    x = make_decode(w, device=device, seed=seed, nan_pad=nan_pad, lens=lens)
    seed = SEEDS.get(w.name, 1) if seed is None else seed
    x["q"] = randn((w.B, w.H_q, w.T_q, w.d), w.torch_dtype, device, seed, 3)
    return x


def make_decode_paged(w: Workload, page_size: int, device="cpu", seed=None, spare_pages=3):
    """Paged-cache decode inputs: the contiguous inputs of ``make_decode_multi``
    (same seeds, so the same values) scattered into a pool of pages.

    Pages are ``[num_pages, H_kv, page_size, d]``; each sequence's logical
    pages take physical pages in a seeded random order, and ``spare_pages``
    extra pages are filled with NaN.  Table entries past a sequence's pages
    name a NaN page (never a page out of range), and rows of a last page
    past the sequence's length are NaN, so a kernel that reads them poisons
    its output.  Returns q, k_pages, v_pages, block_table ``[B, max_pages]``
    int32, kv_lens int32 and the contiguous k, v.
    """
    x = make_decode_multi(w, device=device, seed=seed)
    seed = SEEDS.get(w.name, 1) if seed is None else seed
    k_pages, v_pages, table = scatter_pages(w, x["k"], x["v"], page_size, seed, spare_pages, device)
    return {"q": x["q"], "k_pages": k_pages, "v_pages": v_pages,
            "block_table": table, "kv_lens": x["kv_lens"], "k": x["k"], "v": x["v"]}


def scatter_pages(w: Workload, k, v, page_size: int, seed: int, spare_pages: int, device):
    """Contiguous caches ``[B,H_kv,kv_cap,d]`` scattered into a pool of pages
    ``[num_pages,H_kv,page_size,d]``: each sequence's logical pages take
    physical pages in a seeded random order (generator ``seed*16 + 4``),
    ``spare_pages`` extra pages are NaN, table entries past a sequence's
    pages name a NaN page, and rows of a last page past the length are NaN.
    The pools are built on the host and uploaded with one copy each (no
    per-page device copies).  Returns the K and V pools and the block table
    ``[B, max_pages]`` int32."""
    max_pages = (w.kv_cap + page_size - 1) // page_size
    need = [(L + page_size - 1) // page_size for L in w.lens]
    num_pages = sum(need) + spare_pages
    g = torch.Generator().manual_seed(seed * 16 + 4)
    perm = torch.randperm(num_pages, generator=g)
    nan_page = int(perm[-1])
    table = torch.full((w.B, max_pages), nan_page, dtype=torch.int32)
    pools = []
    for src in (k, v):
        src = src.cpu()
        pool = torch.full((num_pages, w.H_kv, page_size, w.d), float("nan"), dtype=w.torch_dtype)
        nxt = 0
        for b, L in enumerate(w.lens):
            n = need[b]
            phys = perm[nxt:nxt + n]
            nxt += n
            table[b, :n] = phys.to(torch.int32)
            # The sequence's rows, NaN from its length to the end of its last page.
            rows = torch.full((w.H_kv, n * page_size, w.d), float("nan"), dtype=w.torch_dtype)
            rows[:, :L] = src[b, :, :L]
            pool[phys] = rows.reshape(w.H_kv, n, page_size, w.d).transpose(0, 1)
        pools.append(pool.to(device))
    return pools[0], pools[1], table.to(device)


def make_prefill_paged(w: Workload, page_size: int, device="cpu", seed=None, spare_pages=3):
    """Paged-cache varlen prefill inputs: the inputs of ``make_prefill_varlen``
    (same seeds, so the same values) with K/V scattered as by
    ``scatter_pages``.  Returns q, k_pages, v_pages, block_table,
    cu_seqlens_q, kv_lens and the contiguous k, v."""
    x = make_prefill_varlen(w, device=device, seed=seed)
    seed = SEEDS.get(w.name, 1) if seed is None else seed
    k_pages, v_pages, table = scatter_pages(w, x["k"], x["v"], page_size, seed, spare_pages, device)
    x.update({"k_pages": k_pages, "v_pages": v_pages, "block_table": table})
    return x


def make_prefill(w: Workload, device="cpu", seed=None, nan_pad=True, kv_cap=None):
    """Prefill inputs: q ``[B,H_q,S_q,d]``, k/v ``[B,H_kv,kv_cap,d]``."""
    seed = SEEDS.get(w.name, 1) if seed is None else seed
    cap = w.S_kv if kv_cap is None else kv_cap
    dt = w.torch_dtype
    q = randn((w.B, w.H_q, w.S_q, w.d), dt, device, seed, 0)
    k = randn((w.B, w.H_kv, cap, w.d), dt, device, seed, 1)
    v = randn((w.B, w.H_kv, cap, w.d), dt, device, seed, 2)
    if nan_pad and cap > w.S_kv:
        k[:, :, w.S_kv:].fill_(float("nan"))
        v[:, :, w.S_kv:].fill_(float("nan"))
    return {"q": q, "k": k, "v": v}


def make_prefill_varlen(w: Workload, device="cpu", seed=None, nan_pad=True, q_lens=None,
                        lens=None):
    """Varlen prefill inputs: q ``[total_q,H_q,d]`` token-packed (chunk b at
    rows ``cu_seqlens_q[b] ..``), k/v ``[B,H_kv,kv_cap,d]`` NaN past each
    sequence's length, cu_seqlens_q ``[B+1]`` and kv_lens ``[B]`` int32."""
    seed = SEEDS.get(w.name, 1) if seed is None else seed
    q_lens = tuple(w.q_lens) if q_lens is None else tuple(q_lens)
    lens = tuple(w.lens) if lens is None else tuple(lens)
    dt = w.torch_dtype
    cu = [0]
    for sq in q_lens:
        cu.append(cu[-1] + sq)
    q = randn((cu[-1], w.H_q, w.d), dt, device, seed, 0)
    k = randn((w.B, w.H_kv, w.kv_cap, w.d), dt, device, seed, 1)
    v = randn((w.B, w.H_kv, w.kv_cap, w.d), dt, device, seed, 2)
    if nan_pad:
        for b, L in enumerate(lens):
            if L < w.kv_cap:
                k[b, :, L:].fill_(float("nan"))
                v[b, :, L:].fill_(float("nan"))
    return {"q": q, "k": k, "v": v,
            "cu_seqlens_q": torch.tensor(cu, dtype=torch.int32, device=device),
            "kv_lens": torch.tensor(lens, dtype=torch.int32, device=device)}


def sample_rows(S_q: int, n: int, seed: int, always=(0, 1, 63, 64, 127, 128)):
    """Seeded sample of ``n`` distinct query positions in ``[0, S_q)``.

    Always includes the listed tile-edge positions (when in range) and the
    last row, then fills up uniformly without replacement.
    """
    fixed = sorted({r for r in tuple(always) + (S_q - 1,) if 0 <= r < S_q})
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(S_q, generator=g).tolist()
    out = list(fixed)
    seen = set(fixed)
    for r in perm:
        if len(out) >= n:
            break
        if r not in seen:
            out.append(r)
            seen.add(r)
    return sorted(out[:n])


def sample_rows_per_block(S_q: int, n: int, seed: int, block: int = 32,
                          always=(0, 1, 63, 64, 127, 128)):
    """Seeded sample of ``n`` distinct query positions that holds one seeded
    position in every ``block``-position block of ``[0, S_q)`` (so every
    block of rows that one wave of a prefill workgroup owns is represented),
    the listed tile-edge positions and the last row, filled up uniformly
    without replacement."""
    g = torch.Generator().manual_seed(seed)
    nblk = (S_q + block - 1) // block
    off = torch.randint(0, block, (nblk,), generator=g).tolist()
    picked = {min(b * block + o, S_q - 1) for b, o in enumerate(off)}
    picked |= {r for r in tuple(always) + (S_q - 1,) if 0 <= r < S_q}
    if len(picked) > n:
        raise ValueError(f"{len(picked)} required rows exceed the sample size {n}")
    for r in torch.randperm(S_q, generator=g).tolist():
        if len(picked) >= n:
            break
        picked.add(r)
    return sorted(picked)
