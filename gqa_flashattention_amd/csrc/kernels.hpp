// Kernel parameter blocks and launchers shared between the HIP kernels and
// the C-ABI host code.  Plain structs passed by value as kernel arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

struct DecodeParams {
  const void* q;        // [B, H_q, T_q, d]
  const void* k;        // [B, H_kv, kv_cap, d]
  const void* v;        // [B, H_kv, kv_cap, d]
  const int32_t* kv_lens;  // [B] device (used as min(kv_lens[b], max_kv_len))
  void* o;              // [B, H_q, T_q, d]
  float* lse;           // [B, H_q, T_q] or null
  float* ws_o;          // [B, H_q, T_q, n_split_max, d] unnormalised partial O
  float* ws_ml;         // [B, H_q, T_q, n_split_max, 2] partial (m in log2 units, l)
  int B, H_q, H_kv, G, kv_cap;
  int T_q;              // new tokens per sequence (1 for gqa_attn_decode)
  int max_kv_len;
  int chunk;            // keys per split
  int n_split_max;      // ceil(max_kv_len / chunk)
  int q_negate;         // multi-token path: 1 when the scale is negative (Q's sign is flipped)
  float scale_log2;     // scale * log2(e); |scale| * log2(e) on the multi-token path
  // Paged cache (block_table non-null): k, v are [num_pages, H_kv, page, d]
  // pools; position j of sequence b is row j % page of physical page
  // block_table[b * max_pages + j / page]; page = 1 << page_shift.
  const int32_t* block_table;
  int max_pages;
  int page_shift;
  int num_pages;        // pool size; table entries are clamped into [0, num_pages)
  // Fused merge (non-null): [B * H_kv] arrival counters, zero on entry and
  // left zero.  The split kernel's last workgroup of each (sequence, KV
  // head) merges that head's partials itself; no combine launch follows.
  unsigned* counters;
};

struct PrefillParams {
  const void* q;        // [B, H_q, S_q, d]
  const void* k;        // [B, H_kv, kv_cap, d]
  const void* v;        // [B, H_kv, kv_cap, d]
  void* o;              // [B, H_q, S_q, d]
  float* lse;           // [B, H_q, S_q] or null
  int B, H_q, H_kv, G, S_q, S_kv, kv_cap;
  int causal, offset;
  int heads_per_wg;     // query heads of one KV group per workgroup: gcd(G, waves)
  int n_qblk;           // position blocks: ceil(S_q / (32 * waves / heads_per_wg))
  int q_negate;         // 1 when the softmax scale is negative (Q's sign is flipped)
  int pair_blocks;      // dense causal: each workgroup runs a query block and its mirror
  float scale_log2;     // |scale| * log2(e)
  // Varlen batch (both null otherwise): q/o are [S_q = total_q, H_q, d],
  // lse [total_q, H_q]; sequence b's chunk is rows cu_seqlens_q[b] ..
  // cu_seqlens_q[b+1]-1 against min(kv_lens[b], S_kv) keys, causal offset
  // (keys) - (chunk length); n_qblk covers the longest chunk.  `sched`
  // holds B * n_qblk ints: the work list the varlen launch builds first.
  const int* cu_seqlens_q;
  const int* kv_lens;
  int* sched;
  // Paged cache (varlen only; block_table null otherwise): k, v are
  // [num_pages, H_kv, 1 << page_shift, d] pools; position j of sequence b is
  // row j % page of physical page block_table[b * max_pages + j / page].
  const int* block_table;
  int max_pages;
  int page_shift;
  int num_pages;        // pool size; table entries are clamped into [0, num_pages)
};

// Longest block-table row the paged prefill kernel stages in LDS.
constexpr int kPrefillMaxPages = 8192;

struct MergeParams {
  const void* o_a;      // [rows, d]
  const float* lse_a;   // [rows]
  const void* o_b;      // [rows, d]
  const float* lse_b;   // [rows]
  void* o_out;          // [rows, d] (may alias o_a or o_b)
  float* lse_out;       // [rows] or null (may alias lse_a or lse_b)
  long long rows;
};

hipError_t launch_merge(const MergeParams& p, bool bf16, hipStream_t stream);

// Decode launches: the split partial kernel, the combine kernel, or both.
constexpr int kDecodePartial = 1;
constexpr int kDecodeCombine = 2;
constexpr int kDecodeFused = 4;    // with kDecodePartial: the split kernel merges (counters set)
hipError_t launch_decode(const DecodeParams& p, bool bf16, hipStream_t stream, int phases);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);
// Multi-token decode: its partial kernel (chosen by G * T_q) and/or the
// decode combine over the B * H_q * T_q rows.
hipError_t launch_decode_multi(const DecodeParams& p, hipStream_t stream, int phases);
// Row groups of 32 the multi-token partial kernel uses for M = G * T_q rows.
int decode_multi_row_groups(int M);

// Query heads of one KV group a prefill workgroup covers, and the query rows
// (heads x positions) of one workgroup.
int prefill_heads_per_wg(int G);
// Bytes of the varlen prefill work list for B sequences of n_qblk blocks.
inline size_t prefill_varlen_sched_bytes(long long B, long long n_qblk) {
  return (size_t)(((B * n_qblk * 4) + 255) / 256 * 256);
}
int prefill_rows_per_wg();

}  // namespace gqa
