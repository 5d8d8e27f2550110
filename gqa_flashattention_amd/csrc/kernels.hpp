// Kernel parameter blocks and launchers shared between the HIP kernels and
// the C-ABI host code.  Plain structs passed by value as kernel arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

struct DecodeParams {
  const void* q;        // [B, H_q, d]
  const void* k;        // [B, H_kv, kv_cap, d]
  const void* v;        // [B, H_kv, kv_cap, d]
  const int32_t* kv_lens;  // [B] device
  void* o;              // [B, H_q, d]
  float* lse;           // [B, H_q] or null
  float* ws_o;          // [B, H_q, n_split_max, d] unnormalised partial O
  float* ws_ml;         // [B, H_q, n_split_max, 2] partial (m in log2 units, l)
  int B, H_q, H_kv, G, kv_cap;
  int chunk;            // keys per split
  int n_split_max;      // ceil(max_kv_len / chunk)
  float scale_log2;     // scale * log2(e)
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
  float scale_log2;     // |scale| * log2(e)
};

// Decode launches: the split partial kernel, the combine kernel, or both.
constexpr int kDecodePartial = 1;
constexpr int kDecodeCombine = 2;
hipError_t launch_decode(const DecodeParams& p, bool bf16, hipStream_t stream, int phases);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

// Query heads of one KV group a prefill workgroup covers, and the query rows
// (heads x positions) of one workgroup.
int prefill_heads_per_wg(int G);
int prefill_rows_per_wg();

}  // namespace gqa
