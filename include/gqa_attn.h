/*
 * gqa_attn.h -- C ABI of the MI355X (gfx950) grouped-query attention library.
 *
 * Two operations, both exact softmax attention computed FlashAttention-style
 * (tiles of keys folded into a running (m, l, O) state by an online softmax,
 * P.V fused, no score matrix ever written to memory):
 *
 *   gqa_attn_decode   one new query token per sequence (T_q = 1) against a
 *                     read-only K/V cache; FlashDecoding split-KV partials
 *                     merged by a log-sum-exp combine.
 *   gqa_attn_prefill  a chunk of S_q query tokens, optionally causal with an
 *                     offset (the chunk follows causal_offset cached tokens).
 *   gqa_attn_prefill_varlen
 *                     a batch of prefill chunks of different lengths
 *                     (token-packed), each the newest positions of its
 *                     sequence's cache.
 *   gqa_attn_prefill_paged
 *                     the same over a paged K/V cache (block table).
 *   gqa_attn_merge    stitches two (O, lse) results over disjoint key sets.
 *   gqa_attn_decode_paged
 *                     decode (T_q >= 1) over a paged K/V cache (block table).
 *   gqa_attn_decode_multi
 *                     T_q >= 1 new tokens per sequence (speculative or
 *                     short-chunk decode) against the cache that holds them:
 *                     the G heads x T_q tokens of a KV head are M-folded
 *                     into one tile; split-KV partials merged as for decode.
 *
 * Source of the operation: ADR-0060 "AHBM GQA Fused Attention Kernel
 * (Llama3-70B)", kernbench2 revision 5a76ed4: "Algorithm lineage" (exact
 * FlashAttention / FlashDecoding math), §0.5.3 INPUTS and §0.5.4 OUTPUTS (the
 * kernel boundary), §3 "Per-tile op sequence", §4 "Reduction" (the merge),
 * §5.2 (decode is unmasked) and §5.4 (causal tile classes).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers on the current HIP device and
 *    must be 16-byte aligned.  Tensors are dense, row-major, head-major, with
 *    the head dimension d innermost:
 *        q (decode)   [B, H_q, d]          q (prefill)  [B, H_q, S_q, d]
 *        q (decode_multi) [B, H_q, T_q, d]
 *        q (prefill_varlen) [total_q, H_q, d] (token-packed chunks)
 *        k, v cache   [B, H_kv, kv_cap, d] (position j of a sequence = row j)
 *        o            same shape as q, same dtype as q
 *        lse          [B, H_q] (decode) / [B, H_q, S_q] (prefill) /
 *                     [B, H_q, T_q] (decode_multi) / [total_q, H_q]
 *                     (prefill_varlen), float32
 *  - Query head h reads KV head h / (H_q / H_kv): the G = H_q / H_kv query
 *    heads sharing a KV head are adjacent.
 *  - Q and K are already RoPE-rotated, V is raw, and for decode the new
 *    token's K/V row is already in the cache: the library only reads K/V
 *    (preconditions P1-P4 of §0.5.1).
 *  - scale multiplies q.k before the causal mask and the max (softmax_scale
 *    of §0.5.3, normally 1/sqrt(d)).
 *  - lse, when requested, is the natural-log log-sum-exp of the scaled,
 *    visible scores of each query row.
 *  - bf16 inputs are accumulated in float32; the output is rounded to the
 *    input dtype with round-to-nearest-even.
 *
 * Ownership, threading, errors
 * ----------------------------
 *  - The caller owns every buffer (inputs, outputs, workspace).  The library
 *    allocates, frees and synchronises nothing: it validates the arguments,
 *    enqueues kernels on `stream` (a hipStream_t; NULL = the null stream)
 *    and returns.  Entry points are re-entrant; two calls that share a
 *    workspace must not overlap in time.
 *  - Every argument error is reported BEFORE anything is launched, and then
 *    nothing has been written.  Launch failures return GQA_ERR_HIP.
 *    Faults inside a kernel surface at the caller's next synchronisation.
 *  - Values stored in device memory (kv_lens) cannot be checked on the host:
 *    they are a contract (see each entry point).
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQA_DTYPE_F32 = 0,   /* IEEE float32 */
  GQA_DTYPE_BF16 = 1   /* bfloat16 (8-bit exponent, 7-bit mantissa) */
} gqa_dtype_t;

typedef enum {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size or range  */
  GQA_ERR_UNSUPPORTED = 2,  /* valid request the library does not implement */
  GQA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required  */
  GQA_ERR_HIP = 4,          /* the HIP runtime rejected a launch           */
  GQA_ERR_SCRATCH_LIMIT = 5 /* gqa_attn_decode_noalloc: the call needs more
                               than its fixed device scratch               */
} gqa_status_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* gqa_attn_status_string(int status);

/* Version of this library as MAJOR*10000 + MINOR*100 + PATCH. */
int gqa_attn_version(void);

/*
 * Number of keys each decode split (one workgroup's contiguous slice of one
 * sequence) covers for these arguments: `chunk_tokens` itself when it is
 * positive (it must then be a multiple of 128 for bf16, at most 2^20; the
 * f32 path has a fixed split of 64 keys, so for f32 it must be 64), or the library's
 * automatic choice when it is 0.  Splits are contiguous
 * position blocks, the placement the pages require for prefill/decode
 * sharing (§0 "CUBE Group", token-to-rank placement).  Returns a negative
 * gqa_status_t on invalid arguments.
 */
int gqa_attn_decode_split_tokens(int B, int H_kv, int max_kv_len,
                                 int chunk_tokens, int dtype);

/*
 * Device workspace (bytes) gqa_attn_decode needs: a fixed 64 KiB of arrival
 * counters (used only by gqa_attn_decode_fused), then one unnormalised
 * partial (m, l, O[d]) in float32 per (sequence, query head, split), the
 * (m_i, l_i, O_i) of §4.  Returns 0 on invalid arguments.
 */
size_t gqa_attn_decode_workspace_bytes(int B, int H_q, int H_kv, int d,
                                       int max_kv_len, int chunk_tokens,
                                       int dtype);

/*
 * Decode attention, T_q = 1 (§5.2 / §5.3, §4).
 *
 *   q        [B, H_q, d]             dtype
 *   k_cache  [B, H_kv, kv_cap, d]    dtype, read-only
 *   v_cache  [B, H_kv, kv_cap, d]    dtype, read-only
 *   kv_lens  [B] int32, DEVICE memory: sequence b attends to its keys
 *            0 .. kv_lens[b]-1.  Contract (not checked): 1 <= kv_lens[b] <=
 *            max_kv_len.  Cache rows at or past kv_lens[b] are never read,
 *            so they may hold anything (NaN included).  A length above
 *            max_kv_len is read as max_kv_len (nothing past it is read); a
 *            length below 1 leaves that sequence's outputs undefined.
 *   o        [B, H_q, d]             dtype, written
 *   lse      [B, H_q] float32, written when non-NULL
 *   max_kv_len   host-side upper bound of kv_lens, <= kv_cap; it sizes the
 *                launch and the workspace.
 *   chunk_tokens keys per split, 0 = automatic (see above).
 *   workspace    device buffer of at least
 *                gqa_attn_decode_workspace_bytes(...) bytes, 16-byte
 *                aligned; its contents on entry do not matter.  Calls
 *                sharing a workspace must not overlap in time.
 *
 * Two kernel launches on `stream`.  Each workgroup of the first sweeps one
 * split of one (sequence, KV head) with the G query heads folded into the
 * matrix-core tile and writes the unnormalised partial; the second merges
 * the partials of each (sequence, query head) and normalises once.
 * Requirements: d == 128 and G <= 16 (else GQA_ERR_UNSUPPORTED).
 */
int gqa_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* kv_lens, void* o, float* lse,
                    int B, int H_q, int H_kv, int d, int kv_cap,
                    int max_kv_len, float scale, int dtype, int chunk_tokens,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_attn_decode in ONE launch: the data-driven reduction of §4.3 ("no
 * global barrier").  Each split workgroup publishes its partial and counts
 * itself in on its (sequence, KV head)'s arrival counter; the workgroup
 * that arrives last merges that head's partials with the same code and in
 * the same order as the combine launch, so the results are bit-identical
 * to gqa_attn_decode's for the same chunk_tokens.  Same arguments and
 * workspace size as gqa_attn_decode, with one extra contract:
 *
 *  - The arrival counters are the workspace's first 64 KiB (one uint32 per
 *    (sequence, KV head); B * H_kv <= 16384, else GQA_ERR_UNSUPPORTED).
 *    They must be zero before the workspace's FIRST fused call -- zero-fill
 *    it once when it is allocated -- and every fused call leaves them zero
 *    again; no decode entry point writes them otherwise, whatever the
 *    shape, so one workspace serves fused and two-launch calls of any
 *    shape.  After a call that did not complete (a fault), zero it again.
 *  - Calls sharing a workspace must not overlap in time (as for
 *    gqa_attn_decode).
 *
 * Cost on MI355X: the partials are published with write-through
 * (agent-scope) stores, each workgroup waits for their acknowledgement and
 * counts in with one atomic, and the last arriver invalidates its caches
 * before merging -- the other splits may have run on any of the 8 XCDs,
 * whose L2 caches are separate.  Measured, that tail costs more than the
 * second launch of gqa_attn_decode at every size tried (a 256-key fp32
 * call, a 32K-key call, the 8K-128K ragged batch), so gqa_attn_decode stays
 * the faster default; this entry point is for callers that want exactly
 * one kernel per decode step.
 */
int gqa_attn_decode_fused(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* kv_lens, void* o, float* lse,
                          int B, int H_q, int H_kv, int d, int kv_cap,
                          int max_kv_len, float scale, int dtype, int chunk_tokens,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_attn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, the same kernels and the same
 * results bit for bit.  The split partials live in a fixed device array of
 * GQA_DECODE_NOALLOC_SCRATCH_BYTES bytes that the library's code object
 * holds on every device it is loaded on, until the process ends; its device
 * address is looked up once per device, on the first call made with that
 * device current (hipGetSymbolAddress, no allocation).  Nothing in it needs
 * to start at zero: every partial is written before it is read.
 *
 *  - `stream` must belong to the current device (else GQA_ERR_INVALID_ARG).
 *  - A call whose partials would need more than the scratch
 *    (gqa_attn_decode_workspace_bytes(...) > GQA_DECODE_NOALLOC_SCRATCH_BYTES)
 *    returns GQA_ERR_SCRATCH_LIMIT before launching anything.  The limit
 *    holds, for example, B = 4 sequences of up to 131072 keys at H_q = 64
 *    with the automatic split.
 *  - All calls on one device share its scratch: calls that overlap in time
 *    on one device (two streams, or two host threads) race and give wrong
 *    results.  Serialise them.
 *  - It calls no hipMalloc, hipFree or other allocating routine.
 */
#define GQA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

int gqa_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* kv_lens, void* o, float* lse,
                            int B, int H_q, int H_kv, int d, int kv_cap,
                            int max_kv_len, float scale, int dtype, int chunk_tokens,
                            void* stream);

/*
 * The two launches of gqa_attn_decode, separately: _partial runs the split
 * sweeps and writes the partials into `workspace`; _combine merges them
 * into `o` (and `lse`).  Both take exactly the arguments of
 * gqa_attn_decode and validate them the same way; issuing _partial then
 * _combine on one stream with the same arguments is gqa_attn_decode.  For
 * callers that time or schedule the two kernels apart.  _partial does not
 * touch `o`/`lse`; _combine reads only `kv_lens` and the workspace.
 */
int gqa_attn_decode_partial(const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* kv_lens,
                            void* o, float* lse, int B, int H_q, int H_kv,
                            int d, int kv_cap, int max_kv_len, float scale,
                            int dtype, int chunk_tokens, void* workspace,
                            size_t workspace_bytes, void* stream);
int gqa_attn_decode_combine(const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* kv_lens,
                            void* o, float* lse, int B, int H_q, int H_kv,
                            int d, int kv_cap, int max_kv_len, float scale,
                            int dtype, int chunk_tokens, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Multi-token decode: T_q new tokens per sequence (§3 running state of shape
 * [G, T_q]; §5.2 M-fold of the G heads x T_q tokens into the GEMM rows;
 * §0.5.3 q_block_meta {q_start, T_q}; §4 merge).
 *
 *   q        [B, H_q, T_q, d]        bf16: token t of each head is at
 *            position kv_lens[b] - T_q + t of its sequence.
 *   k_cache, v_cache [B, H_kv, kv_cap, d] bf16, read-only, already holding
 *            the T_q new tokens' rows (precondition P3 of §0.5.1).
 *   kv_lens  [B] int32, DEVICE memory: valid length L of each sequence,
 *            new tokens included.  Token t sees keys 0 .. L - T_q + t (a
 *            causal tail: the last T_q - 1 keys are hidden from the earlier
 *            tokens).  Contract (not checked): T_q <= kv_lens[b] <=
 *            max_kv_len.  A length above max_kv_len is read as max_kv_len;
 *            rows of a sequence shorter than T_q get undefined values (no
 *            memory outside the cache rows below max_kv_len is read).
 *   o        [B, H_q, T_q, d] bf16, written
 *   lse      [B, H_q, T_q] float32, written when non-NULL
 *   max_kv_len, chunk_tokens, workspace: as for gqa_attn_decode, with the
 *            sizes from the two functions below.
 *
 * Two kernel launches on `stream`.  Each workgroup of the first folds one
 * split of one (sequence, KV head) into all G*T_q rows -- for G*T_q <= 16
 * with gqa_attn_decode's split kernel (the rows fill its 16-row tile),
 * otherwise with a kernel that stages the split's K/V tiles in LDS for up
 * to four 32-row groups; the second is the decode combine over the
 * B*H_q*T_q rows.
 * Requirements: dtype == GQA_DTYPE_BF16, d == 128 and G*T_q <= 128 (else
 * GQA_ERR_UNSUPPORTED); 1 <= T_q <= max_kv_len <= kv_cap (else
 * GQA_ERR_INVALID_ARG).  T_q == 1 is plain decode (same results within
 * rounding as gqa_attn_decode, through this kernel).
 */
int gqa_attn_decode_multi(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* kv_lens, void* o, float* lse, int B, int H_q,
                          int H_kv, int d, int T_q, int kv_cap, int max_kv_len, float scale,
                          int dtype, int chunk_tokens, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Keys per multi-token decode split: `chunk_tokens` when positive (a
 * multiple of 128, at most 2^20), else the library's automatic choice (it depends on
 * G * T_q, hence H_q).  Returns a negative gqa_status_t on invalid
 * arguments (GQA_ERR_UNSUPPORTED for f32).
 */
int gqa_attn_decode_multi_split_tokens(int B, int H_q, int H_kv, int T_q, int max_kv_len,
                                       int chunk_tokens, int dtype);

/*
 * Device workspace (bytes) gqa_attn_decode_multi needs: one (m, l, O[d])
 * float32 partial per (sequence, query head, token, split).  Returns 0 on
 * invalid or unsupported arguments.
 */
size_t gqa_attn_decode_multi_workspace_bytes(int B, int H_q, int H_kv, int d, int T_q,
                                             int max_kv_len, int chunk_tokens, int dtype);

/*
 * The two launches of gqa_attn_decode_multi separately (as
 * gqa_attn_decode_partial / _combine are for decode): same arguments and
 * validation; _partial then _combine on one stream is gqa_attn_decode_multi.
 */
int gqa_attn_decode_multi_partial(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* kv_lens, void* o, float* lse, int B,
                                  int H_q, int H_kv, int d, int T_q, int kv_cap,
                                  int max_kv_len, float scale, int dtype, int chunk_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream);
int gqa_attn_decode_multi_combine(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* kv_lens, void* o, float* lse, int B,
                                  int H_q, int H_kv, int d, int T_q, int kv_cap,
                                  int max_kv_len, float scale, int dtype, int chunk_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode (T_q >= 1 new tokens per sequence, as gqa_attn_decode_multi; T_q = 1
 * is plain decode) over a paged K/V cache.
 *
 *   k_pages, v_pages [num_pages, H_kv, page_size, d] bf16: a pool of pages,
 *            each holding page_size consecutive positions of every KV head.
 *   block_table [B, max_pages_per_seq] int32, DEVICE memory: position j of
 *            sequence b is row j % page_size of page block_table[b][j /
 *            page_size].  Entries for pages past a sequence's length are
 *            never read.  Contract (not checked): entries lie in
 *            [0, num_pages); an entry outside is read as the nearest end of
 *            that range (wrong values, no memory outside the pool is read).
 *   kv_lens, q, o, lse, max_kv_len, scale, chunk_tokens, workspace: as for
 *            gqa_attn_decode_multi; rows of a sequence's last page past its
 *            length are never read.
 *   page_size  a power of two in [16, 65536]; max_pages_per_seq * page_size
 *            >= max_kv_len.
 *
 * The same two launches as gqa_attn_decode_multi (the split kernel for the
 * fold's size, then the combine); the split kernels address each 16-key
 * sub-block (decode kernel) or 4-row load (multi-token kernel) in its own
 * page, so pages need no particular placement in the pool.  Splits are
 * capped so that one wave range spans at most 64 pages (G*T_q <= 16) or one
 * split at most 128 pages (larger folds): an explicit chunk_tokens above
 * that is GQA_ERR_INVALID_ARG.  Requirements as for gqa_attn_decode_multi
 * (bf16, d == 128, G*T_q <= 128).
 */
int gqa_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                          const int32_t* block_table, const int32_t* kv_lens, void* o,
                          float* lse, int B, int H_q, int H_kv, int d, int T_q, int page_size,
                          int max_pages_per_seq, int num_pages, int max_kv_len, float scale,
                          int dtype, int chunk_tokens, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Its two launches separately, as gqa_attn_decode_partial / _combine are for
 * decode: same arguments and validation; _partial then _combine on one
 * stream is gqa_attn_decode_paged. */
int gqa_attn_decode_paged_partial(const void* q, const void* k_pages, const void* v_pages,
                                  const int32_t* block_table, const int32_t* kv_lens, void* o,
                                  float* lse, int B, int H_q, int H_kv, int d, int T_q,
                                  int page_size, int max_pages_per_seq, int num_pages,
                                  int max_kv_len, float scale, int dtype, int chunk_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream);
int gqa_attn_decode_paged_combine(const void* q, const void* k_pages, const void* v_pages,
                                  const int32_t* block_table, const int32_t* kv_lens, void* o,
                                  float* lse, int B, int H_q, int H_kv, int d, int T_q,
                                  int page_size, int max_pages_per_seq, int num_pages,
                                  int max_kv_len, float scale, int dtype, int chunk_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Keys per split and workspace bytes of gqa_attn_decode_paged (negative
 * status / 0 on invalid arguments, as for the other sizing queries). */
int gqa_attn_decode_paged_split_tokens(int B, int H_q, int H_kv, int T_q, int page_size,
                                       int max_kv_len, int chunk_tokens, int dtype);
size_t gqa_attn_decode_paged_workspace_bytes(int B, int H_q, int H_kv, int d, int T_q,
                                             int page_size, int max_kv_len, int chunk_tokens,
                                             int dtype);

/*
 * Stitching of two attention results for the same query rows over disjoint
 * key sets (a prefix and a chunk, or two KV shards): the log-sum-exp merge
 * of §4 applied to normalised results (each (O, lse) is the partial
 * (m, l, O) = (lse, 1, O)).
 *
 *   o_a, o_b  [rows, d] dtype, with their LSEs lse_a, lse_b [rows] float32
 *             (natural log, as this library exports them).  A row whose lse
 *             is -inf (no visible key on that side) contributes nothing; its
 *             O is not read into the sum (it may hold anything, NaN included).
 *   o_out     [rows, d] dtype, written: (w_a O_a + w_b O_b) / (w_a + w_b)
 *             with w = exp(lse - max(lse_a, lse_b)); rows empty on both
 *             sides get O = 0.  May be the same buffer as o_a or o_b.
 *   lse_out   [rows] float32, written when non-NULL: the merged LSE (-inf
 *             for rows empty on both sides).  May be lse_a or lse_b.
 *
 * One kernel launch on `stream`; arithmetic in float32, output rounded to
 * dtype (RNE).  Requirements: d == 128 (else GQA_ERR_UNSUPPORTED); rows >= 0
 * (0 launches nothing).
 */
int gqa_attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                   void* o_out, float* lse_out, long long rows, int d, int dtype, void* stream);

/*
 * Prefill attention over a chunk of S_q queries (§5.4).
 *
 *   q     [B, H_q, S_q, d]       bf16
 *   k, v  [B, H_kv, kv_cap, d]   bf16, read-only; rows 0 .. S_kv-1 are used
 *   o     [B, H_q, S_q, d]       bf16, written
 *   lse   [B, H_q, S_q] float32, written when non-NULL
 *   causal = 1: query i sees keys j <= causal_offset + i (the chunk follows
 *           causal_offset cached tokens); tiles wholly above the diagonal
 *           are skipped, tiles wholly below are unmasked.  Requires
 *           0 <= causal_offset and causal_offset + S_q <= S_kv.
 *   causal = 0: every query sees all S_kv keys (causal_offset ignored).
 *
 * Requirements: dtype == GQA_DTYPE_BF16 and d == 128 (else
 * GQA_ERR_UNSUPPORTED); S_kv <= kv_cap.
 */
int gqa_attn_prefill(const void* q, const void* k, const void* v, void* o,
                     float* lse, int B, int H_q, int H_kv, int d, int S_q,
                     int S_kv, int kv_cap, int causal, int causal_offset,
                     float scale, int dtype, void* stream);

/*
 * Varlen prefill: chunks of different lengths for B sequences in one launch
 * (chunked prefill / continuous batching).  Each chunk is the newest S_q_b
 * positions of its sequence, whose K/V rows are already in the cache
 * (precondition P3 of §0.5.1), so its query block starts at
 * q_start = kv_lens[b] - S_q_b (q_block_meta of §0.5.3), per sequence.
 *
 *   q     [total_q, H_q, d] bf16, token-packed: sequence b's chunk is rows
 *         cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (token-major, heads inner)
 *   cu_seqlens_q  [B+1] int32 DEVICE array, 4-byte aligned: 0 =
 *         cu_seqlens_q[0] <= cu_seqlens_q[1] <= ... <= cu_seqlens_q[B] =
 *         total_q; a sequence may have an empty chunk
 *   k, v  [B, H_kv, kv_cap, d] bf16, read-only
 *   kv_lens       [B] int32 DEVICE array, 4-byte aligned: valid positions
 *         of each sequence's cache (the chunk included)
 *   o     [total_q, H_q, d] bf16, written
 *   lse   [total_q, H_q] float32, written when non-NULL
 *   causal = 1: token i of chunk b sees keys j <= kv_lens[b] - S_q_b + i;
 *           requires S_q_b <= kv_lens[b].
 *   causal = 0: every token of chunk b sees all kv_lens[b] keys.
 *   max_seqlen_q  an upper bound of every S_q_b (sizes the grid; rows past
 *         it are not written); max_kv_len an upper bound of every kv_lens[b]
 *         (kv_lens are clamped to it), 1 <= max_kv_len <= kv_cap.
 *
 * The device arrays are not read on the host: values outside the contract
 * are clamped inside the kernel (no access leaves the buffers), but the
 * results for such sequences are meaningless.  A sequence with
 * kv_lens[b] = 0 and a non-empty chunk (non-causal) gets O = 0, lse = -inf.
 *
 *   workspace  DEVICE scratch of at least
 *         gqa_attn_prefill_varlen_workspace_bytes(B, H_q, H_kv, max_seqlen_q)
 *         bytes, 256-byte aligned (else GQA_ERR_WORKSPACE): a first, small
 *         kernel writes the work list there (every (sequence, query block)
 *         ordered by its key-tile count, heaviest first) and the attention
 *         kernel reads it.  Its previous contents do not matter.
 *
 * Two launches on `stream`.  Requirements: dtype == GQA_DTYPE_BF16 and
 * d == 128 (else GQA_ERR_UNSUPPORTED); 0 <= max_seqlen_q <= total_q
 * (total_q = 0 or max_seqlen_q = 0 launches nothing and needs no workspace).
 */
int gqa_attn_prefill_varlen(const void* q, const void* k, const void* v,
                            const int* cu_seqlens_q, const int* kv_lens, void* o,
                            float* lse, int B, int H_q, int H_kv, int d, int total_q,
                            int max_seqlen_q, int kv_cap, int max_kv_len, int causal,
                            float scale, int dtype, void* workspace,
                            size_t workspace_bytes, void* stream);
/* Workspace bytes gqa_attn_prefill_varlen needs; 0 for invalid sizes. */
size_t gqa_attn_prefill_varlen_workspace_bytes(int B, int H_q, int H_kv, int max_seqlen_q);

/*
 * Varlen prefill over a paged K/V cache: gqa_attn_prefill_varlen with the
 * cache in a page pool addressed through a block table (the driver-chosen
 * placement of each KV block, §2.1, made explicit).  Same q, o, lse,
 * cu_seqlens_q, kv_lens, causal, max_seqlen_q, scale and workspace (its
 * size from gqa_attn_prefill_varlen_workspace_bytes) as there.
 *
 *   k_pages, v_pages  [num_pages, H_kv, page_size, d] bf16 pools, read-only:
 *         position j of sequence b is row j % page_size of physical page
 *         block_table[b * max_pages_per_seq + j / page_size]
 *   block_table  [B, max_pages_per_seq] int32 DEVICE array, 4-byte aligned.
 *         Entries outside [0, num_pages) are clamped into the pool (wrong
 *         values, never an access outside it); entries past a sequence's
 *         pages are not read.
 *   page_size    a power of two, 16 .. 65536
 *   max_kv_len   an upper bound of every kv_lens[b] (clamped to it),
 *         1 <= max_kv_len <= max_pages_per_seq * page_size
 *
 * Requirements as for gqa_attn_prefill_varlen, and at most 8192 pages per
 * sequence (ceil(max_kv_len / page_size) <= 8192, else GQA_ERR_UNSUPPORTED:
 * the kernel stages a sequence's table row in LDS).
 */
int gqa_attn_prefill_paged(const void* q, const void* k_pages, const void* v_pages,
                           const int* block_table, const int* cu_seqlens_q,
                           const int* kv_lens, void* o, float* lse, int B, int H_q,
                           int H_kv, int d, int total_q, int max_seqlen_q, int page_size,
                           int max_pages_per_seq, int num_pages, int max_kv_len,
                           int causal, float scale, int dtype, void* workspace,
                           size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
