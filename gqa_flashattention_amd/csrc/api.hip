// C-ABI entry points: host-side argument validation, work decomposition and
// kernel launches.  Declarations and the full contract are in
// include/gqa_attn.h.  Nothing here allocates, frees or synchronises.

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "gqa_attn.h"
#include "kernels.hpp"

namespace {

constexpr int kD = 128;
constexpr int kMaxG = 16;          // query heads per KV head the decode MFMA tile holds
constexpr int kF32Chunk = 64;      // keys per split of the fp32 decode path
constexpr int kBf16ChunkQuantum = 128;  // 4 waves x 32-key blocks
// Largest explicit split: keeps every per-wave and per-split byte count of
// the split kernels' 32-bit buffer resources and offsets far from overflow.
constexpr int kMaxChunk = 1 << 20;
constexpr int kMultiMaxRows = 128;      // G * T_q rows of the multi-token decode tile
constexpr size_t kWsAlign = 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Effective keys per decode split, or a negative status.
int split_tokens(int B, int H_kv, int max_kv_len, int chunk_tokens, int dtype) {
  if (B < 1 || H_kv < 1 || max_kv_len < 1 || chunk_tokens < 0) return -GQA_ERR_INVALID_ARG;
  if (dtype == GQA_DTYPE_F32) {
    if (chunk_tokens != 0 && chunk_tokens != kF32Chunk) return -GQA_ERR_INVALID_ARG;
    return kF32Chunk;
  }
  if (dtype != GQA_DTYPE_BF16) return -GQA_ERR_INVALID_ARG;
  if (chunk_tokens > 0) {
    if (chunk_tokens % kBf16ChunkQuantum != 0 || chunk_tokens > kMaxChunk) return -GQA_ERR_INVALID_ARG;
    return chunk_tokens;
  }
  // About 64 splits of the longest sequence, in multiples of 128 keys,
  // between 256 and 1280 keys.  Measured on MI355X: 512 keys is best for one
  // 32K-key sequence (partial traffic and the combine stay small), 1280 for
  // a ragged batch up to 128K keys (more workgroups keep HBM busy).
  long long c = ((long long)max_kv_len + 63) / 64;
  c = (c + kBf16ChunkQuantum - 1) / kBf16ChunkQuantum * kBf16ChunkQuantum;
  if (c < 2 * kBf16ChunkQuantum) c = 2 * kBf16ChunkQuantum;
  if (c > 10 * kBf16ChunkQuantum) c = 10 * kBf16ChunkQuantum;
  const long long cap = ((long long)max_kv_len + kBf16ChunkQuantum - 1) / kBf16ChunkQuantum * kBf16ChunkQuantum;
  if (c > cap) c = cap;
  return (int)c;
}

// A multi-token decode whose G * T_q folded rows fit the decode kernel's
// 16-row tile runs on the decode split kernel; larger folds run on the
// multi-token kernel.
bool multi_on_decode_kernel(int G, int T_q) { return (long long)G * T_q <= kMaxG; }

// Effective keys per multi-token decode split, or a negative status.
int multi_split_tokens(int B, int H_q, int H_kv, int T_q, int max_kv_len, int chunk_tokens,
                       int dtype) {
  if (B < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || T_q < 1 || max_kv_len < 1 ||
      chunk_tokens < 0)
    return -GQA_ERR_INVALID_ARG;
  if (T_q > max_kv_len) return -GQA_ERR_INVALID_ARG;
  if (dtype == GQA_DTYPE_F32) return -GQA_ERR_UNSUPPORTED;
  if (dtype != GQA_DTYPE_BF16) return -GQA_ERR_INVALID_ARG;
  if (multi_on_decode_kernel(H_q / H_kv, T_q))
    return split_tokens(B, H_kv, max_kv_len, chunk_tokens, dtype);
  if (chunk_tokens > 0) {
    if (chunk_tokens % kBf16ChunkQuantum != 0 || chunk_tokens > kMaxChunk) return -GQA_ERR_INVALID_ARG;
    return chunk_tokens;
  }
  // About 32 splits of the longest sequence, in multiples of 128 keys,
  // between 256 and 2048 keys: one 32K-key sequence then fills the 256 CUs
  // with one workgroup each, and a split's partial (G * T_q rows of d + 2
  // floats) stays small against the K/V it covers.
  long long c = ((long long)max_kv_len + 31) / 32;
  c = (c + kBf16ChunkQuantum - 1) / kBf16ChunkQuantum * kBf16ChunkQuantum;
  if (c < 2 * kBf16ChunkQuantum) c = 2 * kBf16ChunkQuantum;
  if (c > 16 * kBf16ChunkQuantum) c = 16 * kBf16ChunkQuantum;
  const long long cap = ((long long)max_kv_len + kBf16ChunkQuantum - 1) / kBf16ChunkQuantum * kBf16ChunkQuantum;
  if (c > cap) c = cap;
  return (int)c;
}

// log2 of a paged-cache page size, or -1 unless it is a power of two in
// [16, 65536].
int page_shift_of(int page_size) {
  if (page_size < 16 || page_size > 65536 || (page_size & (page_size - 1))) return -1;
  int sh = 0;
  while ((1 << sh) < page_size) ++sh;
  return sh;
}

// Keys per split of a paged-cache decode, or a negative status: the rule of
// the kernel the fold runs on, with splits small enough that the decode
// kernel's wave ranges span at most 64 pages and the multi-token kernel's
// splits at most 128 (each keeps its page numbers in one or two registers).
int paged_split_tokens(int B, int H_q, int H_kv, int T_q, int page_size, int max_kv_len,
                       int chunk_tokens, int dtype) {
  const int sh = page_shift_of(page_size);
  if (sh < 0) return -GQA_ERR_INVALID_ARG;
  int c = multi_split_tokens(B, H_q, H_kv, T_q, max_kv_len, chunk_tokens, dtype);
  if (c <= 0) return c;
  const bool dk = multi_on_decode_kernel(H_q / H_kv, T_q);
  const long long limit = dk ? 4LL * 63 * page_size : 127LL * page_size;   // keys per split
  if (c > limit) {
    if (chunk_tokens > 0) return -GQA_ERR_INVALID_ARG;
    c = (int)(limit / kBf16ChunkQuantum * kBf16ChunkQuantum);
  }
  return c;
}

// Decode workspace: [arrival counters, a fixed 64 KiB] [partial O]
// [partial (m, l)], each region 256-byte aligned.  The counters (one uint32
// per (sequence, KV head), at most kMaxCounters) are written only by the
// fused decode, which leaves them zero; they sit at the same offset for
// every shape, so a workspace zeroed once serves fused calls of any shape
// while partials of any call never land on them.
constexpr size_t kCounterBytes = 64 << 10;
constexpr int kMaxCounters = (int)(kCounterBytes / sizeof(unsigned));

struct WsLayout {
  size_t o_off, ml_off, total;
};

WsLayout ws_layout(int B, int H_q, int n_split) {
  WsLayout w;
  w.o_off = kCounterBytes;
  w.ml_off = w.o_off + round_up((size_t)B * H_q * n_split * kD * sizeof(float), kWsAlign);
  w.total = w.ml_off + round_up((size_t)B * H_q * n_split * 2 * sizeof(float), kWsAlign);
  return w;
}

}  // namespace

extern "C" {

const char* gqa_attn_status_string(int status) {
  switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_INVALID_ARG: return "invalid argument";
    case GQA_ERR_UNSUPPORTED: return "unsupported configuration";
    case GQA_ERR_WORKSPACE: return "workspace missing or too small";
    case GQA_ERR_HIP: return "HIP runtime error at launch";
    case GQA_ERR_SCRATCH_LIMIT: return "request exceeds the fixed scratch of the allocation-free decode";
    default: return "unknown status";
  }
}

int gqa_attn_version(void) { return 220; }

int gqa_attn_decode_split_tokens(int B, int H_kv, int max_kv_len, int chunk_tokens, int dtype) {
  return split_tokens(B, H_kv, max_kv_len, chunk_tokens, dtype);
}

size_t gqa_attn_decode_workspace_bytes(int B, int H_q, int H_kv, int d, int max_kv_len,
                                       int chunk_tokens, int dtype) {
  if (H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || d != kD) return 0;
  const int chunk = split_tokens(B, H_kv, max_kv_len, chunk_tokens, dtype);
  if (chunk <= 0) return 0;
  const int n_split = (max_kv_len + chunk - 1) / chunk;
  return ws_layout(B, H_q, n_split).total;
}

static int decode_phases(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* kv_lens, void* o, float* lse, int B, int H_q, int H_kv,
                         int d, int kv_cap, int max_kv_len, float scale, int dtype,
                         int chunk_tokens, void* workspace, size_t workspace_bytes, void* stream,
                         int phases) {
  if (!q || !k_cache || !v_cache || !kv_lens || !o) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return GQA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(kv_lens) & 3u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return GQA_ERR_INVALID_ARG;
  if (B < 1 || H_q < 1 || H_kv < 1 || d < 1 || kv_cap < 1 || max_kv_len < 1)
    return GQA_ERR_INVALID_ARG;
  if (H_q % H_kv != 0 || max_kv_len > kv_cap) return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16) return GQA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return GQA_ERR_INVALID_ARG;
  if (chunk_tokens < 0) return GQA_ERR_INVALID_ARG;
  if (B > 65535 || H_kv > 65535) return GQA_ERR_INVALID_ARG;
  if (d != kD || H_q / H_kv > kMaxG) return GQA_ERR_UNSUPPORTED;
  if ((phases & gqa::kDecodeFused) && (long long)B * H_kv > kMaxCounters) return GQA_ERR_UNSUPPORTED;
  const int chunk = split_tokens(B, H_kv, max_kv_len, chunk_tokens, dtype);
  if (chunk <= 0) return GQA_ERR_INVALID_ARG;
  const int n_split = (max_kv_len + chunk - 1) / chunk;
  const WsLayout wl = ws_layout(B, H_q, n_split);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 15u)) return GQA_ERR_WORKSPACE;
  if (workspace_bytes < wl.total) return GQA_ERR_WORKSPACE;

  gqa::DecodeParams p;
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.kv_lens = kv_lens;
  p.o = o;
  p.lse = lse;
  p.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.o_off);
  p.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.ml_off);
  p.counters = (phases & gqa::kDecodeFused) ? static_cast<unsigned*>(workspace) : nullptr;
  p.B = B;
  p.H_q = H_q;
  p.H_kv = H_kv;
  p.G = H_q / H_kv;
  p.kv_cap = kv_cap;
  p.T_q = 1;
  p.block_table = nullptr;
  p.max_pages = 0;
  p.page_shift = 0;
  p.num_pages = 0;
  p.max_kv_len = max_kv_len;
  p.chunk = chunk;
  p.n_split_max = n_split;
  p.q_negate = 0;
  p.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = gqa::launch_decode(p, dtype == GQA_DTYPE_BF16, static_cast<hipStream_t>(stream),
                                    phases);
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int gqa_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* kv_lens, void* o, float* lse, int B, int H_q, int H_kv,
                    int d, int kv_cap, int max_kv_len, float scale, int dtype, int chunk_tokens,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return decode_phases(q, k_cache, v_cache, kv_lens, o, lse, B, H_q, H_kv, d, kv_cap, max_kv_len,
                       scale, dtype, chunk_tokens, workspace, workspace_bytes, stream,
                       gqa::kDecodePartial | gqa::kDecodeCombine);
}

}  // extern "C"

namespace {

// The allocation-free decode's partials: a fixed array in the library's
// code object, one copy per device.  Host code never uses its name as an
// address (that is a host-side stand-in); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and kept here.
__device__ __align__(256) unsigned char scratch[GQA_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_of_current_device(void* stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GQA_ERR_HIP;
  if (dev >= kMaxDevices) return GQA_ERR_UNSUPPORTED;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
      return GQA_ERR_INVALID_ARG;
    if (sdev != dev) return GQA_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return GQA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* kv_lens, void* o, float* lse, int B, int H_q,
                            int H_kv, int d, int kv_cap, int max_kv_len, float scale, int dtype,
                            int chunk_tokens, void* stream) {
  // The size rule first (host arithmetic only), so that an oversized call
  // is rejected before any device is touched; decode_phases checks the rest.
  const size_t need =
      gqa_attn_decode_workspace_bytes(B, H_q, H_kv, d, max_kv_len, chunk_tokens, dtype);
  if (need > GQA_DECODE_NOALLOC_SCRATCH_BYTES) return GQA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (need > 0) {
    const int st = scratch_of_current_device(stream, &ws);
    if (st != GQA_OK) return st;
  }
  return decode_phases(q, k_cache, v_cache, kv_lens, o, lse, B, H_q, H_kv, d, kv_cap, max_kv_len,
                       scale, dtype, chunk_tokens, ws, GQA_DECODE_NOALLOC_SCRATCH_BYTES, stream,
                       gqa::kDecodePartial | gqa::kDecodeCombine);
}

int gqa_attn_decode_fused(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* kv_lens, void* o, float* lse, int B, int H_q, int H_kv,
                          int d, int kv_cap, int max_kv_len, float scale, int dtype,
                          int chunk_tokens, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return decode_phases(q, k_cache, v_cache, kv_lens, o, lse, B, H_q, H_kv, d, kv_cap, max_kv_len,
                       scale, dtype, chunk_tokens, workspace, workspace_bytes, stream,
                       gqa::kDecodePartial | gqa::kDecodeFused);
}

int gqa_attn_decode_partial(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* kv_lens, void* o, float* lse, int B, int H_q,
                            int H_kv, int d, int kv_cap, int max_kv_len, float scale, int dtype,
                            int chunk_tokens, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return decode_phases(q, k_cache, v_cache, kv_lens, o, lse, B, H_q, H_kv, d, kv_cap, max_kv_len,
                       scale, dtype, chunk_tokens, workspace, workspace_bytes, stream,
                       gqa::kDecodePartial);
}

int gqa_attn_decode_combine(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* kv_lens, void* o, float* lse, int B, int H_q,
                            int H_kv, int d, int kv_cap, int max_kv_len, float scale, int dtype,
                            int chunk_tokens, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return decode_phases(q, k_cache, v_cache, kv_lens, o, lse, B, H_q, H_kv, d, kv_cap, max_kv_len,
                       scale, dtype, chunk_tokens, workspace, workspace_bytes, stream,
                       gqa::kDecodeCombine);
}

int gqa_attn_decode_multi_split_tokens(int B, int H_q, int H_kv, int T_q, int max_kv_len,
                                       int chunk_tokens, int dtype) {
  return multi_split_tokens(B, H_q, H_kv, T_q, max_kv_len, chunk_tokens, dtype);
}

size_t gqa_attn_decode_multi_workspace_bytes(int B, int H_q, int H_kv, int d, int T_q,
                                             int max_kv_len, int chunk_tokens, int dtype) {
  if (H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || d != kD) return 0;
  if ((long long)(H_q / H_kv) * T_q > kMultiMaxRows) return 0;
  const int chunk = multi_split_tokens(B, H_q, H_kv, T_q, max_kv_len, chunk_tokens, dtype);
  if (chunk <= 0) return 0;
  const int n_split = (max_kv_len + chunk - 1) / chunk;
  return ws_layout(B, H_q * T_q, n_split).total;
}

static int decode_multi_phases(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* kv_lens, void* o, float* lse, int B, int H_q,
                               int H_kv, int d, int T_q, int kv_cap, int max_kv_len, float scale,
                               int dtype, int chunk_tokens, void* workspace,
                               size_t workspace_bytes, void* stream, int phases) {
  if (!q || !k_cache || !v_cache || !kv_lens || !o) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return GQA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(kv_lens) & 3u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return GQA_ERR_INVALID_ARG;
  if (B < 1 || H_q < 1 || H_kv < 1 || d < 1 || T_q < 1 || kv_cap < 1 || max_kv_len < 1)
    return GQA_ERR_INVALID_ARG;
  if (H_q % H_kv != 0 || max_kv_len > kv_cap || T_q > max_kv_len) return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16) return GQA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return GQA_ERR_INVALID_ARG;
  if (chunk_tokens < 0) return GQA_ERR_INVALID_ARG;
  if (B > 65535 || H_kv > 65535) return GQA_ERR_INVALID_ARG;
  if ((long long)B * H_q * T_q > 0x7fffffffLL) return GQA_ERR_INVALID_ARG;
  if (d != kD || dtype != GQA_DTYPE_BF16 || (long long)(H_q / H_kv) * T_q > kMultiMaxRows)
    return GQA_ERR_UNSUPPORTED;
  const int chunk = multi_split_tokens(B, H_q, H_kv, T_q, max_kv_len, chunk_tokens, dtype);
  if (chunk <= 0) return GQA_ERR_INVALID_ARG;
  const int n_split = (max_kv_len + chunk - 1) / chunk;
  const WsLayout wl = ws_layout(B, H_q * T_q, n_split);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 15u)) return GQA_ERR_WORKSPACE;
  if (workspace_bytes < wl.total) return GQA_ERR_WORKSPACE;

  gqa::DecodeParams p;
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.kv_lens = kv_lens;
  p.o = o;
  p.lse = lse;
  p.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.o_off);
  p.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.ml_off);
  p.counters = nullptr;
  p.B = B;
  p.H_q = H_q;
  p.H_kv = H_kv;
  p.G = H_q / H_kv;
  p.kv_cap = kv_cap;
  p.T_q = T_q;
  p.block_table = nullptr;
  p.max_pages = 0;
  p.page_shift = 0;
  p.num_pages = 0;
  p.max_kv_len = max_kv_len;
  p.chunk = chunk;
  p.n_split_max = n_split;
  hipError_t e;
  if (multi_on_decode_kernel(p.G, T_q)) {
    p.q_negate = 0;
    p.scale_log2 = scale * 1.4426950408889634f;   // the decode kernel takes the signed scale
    e = gqa::launch_decode(p, true, static_cast<hipStream_t>(stream), phases);
  } else {
    p.q_negate = scale < 0.f;
    p.scale_log2 = fabsf(scale) * 1.4426950408889634f;
    e = gqa::launch_decode_multi(p, static_cast<hipStream_t>(stream), phases);
  }
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

#define GQA_MULTI_ARGS                                                                        \
  q, k_cache, v_cache, kv_lens, o, lse, B, H_q, H_kv, d, T_q, kv_cap, max_kv_len, scale, dtype, \
      chunk_tokens, workspace, workspace_bytes, stream

int gqa_attn_decode_multi(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* kv_lens, void* o, float* lse, int B, int H_q, int H_kv,
                          int d, int T_q, int kv_cap, int max_kv_len, float scale, int dtype,
                          int chunk_tokens, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return decode_multi_phases(GQA_MULTI_ARGS, gqa::kDecodePartial | gqa::kDecodeCombine);
}

int gqa_attn_decode_multi_partial(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* kv_lens, void* o, float* lse, int B, int H_q,
                                  int H_kv, int d, int T_q, int kv_cap, int max_kv_len,
                                  float scale, int dtype, int chunk_tokens, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return decode_multi_phases(GQA_MULTI_ARGS, gqa::kDecodePartial);
}

int gqa_attn_decode_multi_combine(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* kv_lens, void* o, float* lse, int B, int H_q,
                                  int H_kv, int d, int T_q, int kv_cap, int max_kv_len,
                                  float scale, int dtype, int chunk_tokens, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return decode_multi_phases(GQA_MULTI_ARGS, gqa::kDecodeCombine);
}

#undef GQA_MULTI_ARGS

int gqa_attn_decode_paged_split_tokens(int B, int H_q, int H_kv, int T_q, int page_size,
                                       int max_kv_len, int chunk_tokens, int dtype) {
  return paged_split_tokens(B, H_q, H_kv, T_q, page_size, max_kv_len, chunk_tokens, dtype);
}

size_t gqa_attn_decode_paged_workspace_bytes(int B, int H_q, int H_kv, int d, int T_q,
                                             int page_size, int max_kv_len, int chunk_tokens,
                                             int dtype) {
  if (H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || d != kD) return 0;
  if ((long long)(H_q / H_kv) * T_q > kMultiMaxRows) return 0;
  const int chunk = paged_split_tokens(B, H_q, H_kv, T_q, page_size, max_kv_len, chunk_tokens, dtype);
  if (chunk <= 0) return 0;
  const int n_split = (max_kv_len + chunk - 1) / chunk;
  return ws_layout(B, H_q * T_q, n_split).total;
}

static int decode_paged_phases(const void* q, const void* k_pages, const void* v_pages,
                               const int32_t* block_table, const int32_t* kv_lens, void* o,
                               float* lse, int B, int H_q, int H_kv, int d, int T_q,
                               int page_size, int max_pages_per_seq, int num_pages,
                               int max_kv_len, float scale, int dtype, int chunk_tokens,
                               void* workspace, size_t workspace_bytes, void* stream,
                               int phases) {
  if (!q || !k_pages || !v_pages || !block_table || !kv_lens || !o) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o))
    return GQA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(kv_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return GQA_ERR_INVALID_ARG;
  if (B < 1 || H_q < 1 || H_kv < 1 || d < 1 || T_q < 1 || max_kv_len < 1 || num_pages < 1 ||
      max_pages_per_seq < 1)
    return GQA_ERR_INVALID_ARG;
  if (H_q % H_kv != 0 || T_q > max_kv_len) return GQA_ERR_INVALID_ARG;
  const int sh = page_shift_of(page_size);
  if (sh < 0) return GQA_ERR_INVALID_ARG;
  if ((long long)max_pages_per_seq * page_size < max_kv_len) return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16) return GQA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return GQA_ERR_INVALID_ARG;
  if (chunk_tokens < 0) return GQA_ERR_INVALID_ARG;
  if (B > 65535 || H_kv > 65535) return GQA_ERR_INVALID_ARG;
  if ((long long)B * H_q * T_q > 0x7fffffffLL) return GQA_ERR_INVALID_ARG;
  if (d != kD || dtype != GQA_DTYPE_BF16 || (long long)(H_q / H_kv) * T_q > kMultiMaxRows)
    return GQA_ERR_UNSUPPORTED;
  const int chunk = paged_split_tokens(B, H_q, H_kv, T_q, page_size, max_kv_len, chunk_tokens, dtype);
  if (chunk <= 0) return GQA_ERR_INVALID_ARG;
  const int n_split = (max_kv_len + chunk - 1) / chunk;
  const WsLayout wl = ws_layout(B, H_q * T_q, n_split);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 15u)) return GQA_ERR_WORKSPACE;
  if (workspace_bytes < wl.total) return GQA_ERR_WORKSPACE;

  gqa::DecodeParams p;
  p.q = q;
  p.k = k_pages;
  p.v = v_pages;
  p.kv_lens = kv_lens;
  p.o = o;
  p.lse = lse;
  p.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.o_off);
  p.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.ml_off);
  p.counters = nullptr;
  p.B = B;
  p.H_q = H_q;
  p.H_kv = H_kv;
  p.G = H_q / H_kv;
  p.kv_cap = 0;
  p.T_q = T_q;
  p.block_table = block_table;
  p.max_pages = max_pages_per_seq;
  p.page_shift = sh;
  p.num_pages = num_pages;
  p.max_kv_len = max_kv_len;
  p.chunk = chunk;
  p.n_split_max = n_split;
  hipError_t e;
  if (multi_on_decode_kernel(p.G, T_q)) {
    p.q_negate = 0;
    p.scale_log2 = scale * 1.4426950408889634f;
    e = gqa::launch_decode(p, true, static_cast<hipStream_t>(stream), phases);
  } else {
    p.q_negate = scale < 0.f;
    p.scale_log2 = fabsf(scale) * 1.4426950408889634f;
    e = gqa::launch_decode_multi(p, static_cast<hipStream_t>(stream), phases);
  }
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

#define GQA_PAGED_ARGS                                                                       \
  q, k_pages, v_pages, block_table, kv_lens, o, lse, B, H_q, H_kv, d, T_q, page_size,          \
      max_pages_per_seq, num_pages, max_kv_len, scale, dtype, chunk_tokens, workspace,           \
      workspace_bytes, stream
#define GQA_PAGED_PARAMS                                                                     \
  const void *q, const void *k_pages, const void *v_pages, const int32_t *block_table,         \
      const int32_t *kv_lens, void *o, float *lse, int B, int H_q, int H_kv, int d, int T_q,      \
      int page_size, int max_pages_per_seq, int num_pages, int max_kv_len, float scale,         \
      int dtype, int chunk_tokens, void *workspace, size_t workspace_bytes, void *stream

int gqa_attn_decode_paged(GQA_PAGED_PARAMS) {
  return decode_paged_phases(GQA_PAGED_ARGS, gqa::kDecodePartial | gqa::kDecodeCombine);
}
int gqa_attn_decode_paged_partial(GQA_PAGED_PARAMS) {
  return decode_paged_phases(GQA_PAGED_ARGS, gqa::kDecodePartial);
}
int gqa_attn_decode_paged_combine(GQA_PAGED_PARAMS) {
  return decode_paged_phases(GQA_PAGED_ARGS, gqa::kDecodeCombine);
}

#undef GQA_PAGED_ARGS
#undef GQA_PAGED_PARAMS

int gqa_attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                   void* o_out, float* lse_out, long long rows, int d, int dtype, void* stream) {
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out) return GQA_ERR_INVALID_ARG;
  if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o_out)) return GQA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(lse_a) & 3u) || (reinterpret_cast<uintptr_t>(lse_b) & 3u) ||
      (reinterpret_cast<uintptr_t>(lse_out) & 3u))
    return GQA_ERR_INVALID_ARG;
  if (rows < 0 || d < 1) return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16) return GQA_ERR_INVALID_ARG;
  if (d != kD) return GQA_ERR_UNSUPPORTED;
  if (rows > (1LL << 34)) return GQA_ERR_INVALID_ARG;
  if (rows == 0) return GQA_OK;
  gqa::MergeParams p;
  p.o_a = o_a;
  p.lse_a = lse_a;
  p.o_b = o_b;
  p.lse_b = lse_b;
  p.o_out = o_out;
  p.lse_out = lse_out;
  p.rows = rows;
  hipError_t e = gqa::launch_merge(p, dtype == GQA_DTYPE_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int gqa_attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H_q, int H_kv, int d, int S_q, int S_kv, int kv_cap, int causal,
                     int causal_offset, float scale, int dtype, void* stream) {
  if (!q || !k || !v || !o) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return GQA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return GQA_ERR_INVALID_ARG;
  if (B < 1 || H_q < 1 || H_kv < 1 || d < 1 || S_q < 1 || S_kv < 1 || kv_cap < 1)
    return GQA_ERR_INVALID_ARG;
  if (H_q % H_kv != 0 || S_kv > kv_cap) return GQA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return GQA_ERR_INVALID_ARG;
  if (causal && (causal_offset < 0 || (long long)causal_offset + S_q > S_kv))
    return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16) return GQA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return GQA_ERR_INVALID_ARG;
  if (d != kD || dtype != GQA_DTYPE_BF16) return GQA_ERR_UNSUPPORTED;
  const int hpw = gqa::prefill_heads_per_wg(H_q / H_kv);
  const long long rows_per_wg = gqa::prefill_rows_per_wg() / hpw;
  const long long n_qblk = ((long long)S_q + rows_per_wg - 1) / rows_per_wg;
  if (n_qblk * B * H_kv * ((H_q / H_kv) / hpw) > 0x7fffffffLL) return GQA_ERR_INVALID_ARG;

  gqa::PrefillParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.H_q = H_q;
  p.H_kv = H_kv;
  p.G = H_q / H_kv;
  p.S_q = S_q;
  p.S_kv = S_kv;
  p.kv_cap = kv_cap;
  p.causal = causal;
  p.offset = causal ? causal_offset : 0;
  p.heads_per_wg = hpw;
  p.n_qblk = (int)n_qblk;
  p.q_negate = scale < 0.f;
  p.pair_blocks = causal ? 1 : 0;
  p.scale_log2 = fabsf(scale) * 1.4426950408889634f;
  p.cu_seqlens_q = nullptr;
  p.kv_lens = nullptr;
  p.sched = nullptr;
  hipError_t e = gqa::launch_prefill(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

size_t gqa_attn_prefill_varlen_workspace_bytes(int B, int H_q, int H_kv, int max_seqlen_q) {
  if (B < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || max_seqlen_q < 0) return 0;
  const int hpw = gqa::prefill_heads_per_wg(H_q / H_kv);
  const long long rows_per_wg = gqa::prefill_rows_per_wg() / hpw;
  const long long n_qblk = ((long long)max_seqlen_q + rows_per_wg - 1) / rows_per_wg;
  return gqa::prefill_varlen_sched_bytes(B, n_qblk);
}

// Varlen prefill on a contiguous cache (block_table null) or a paged one.
static int prefill_varlen_common(const void* q, const void* k, const void* v,
                                 const int* cu_seqlens_q, const int* kv_lens, void* o, float* lse,
                                 int B, int H_q, int H_kv, int d, int total_q, int max_seqlen_q,
                                 int kv_cap, int max_kv_len, int causal, float scale, int dtype,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 const int* block_table, int page_shift, int max_pages,
                                 int num_pages) {
  if (!q || !k || !v || !o || !cu_seqlens_q || !kv_lens) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return GQA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(cu_seqlens_q) |
       reinterpret_cast<uintptr_t>(kv_lens)) & 3u)
    return GQA_ERR_INVALID_ARG;
  if (B < 1 || H_q < 1 || H_kv < 1 || d < 1 || total_q < 0 || kv_cap < 1)
    return GQA_ERR_INVALID_ARG;
  if (max_seqlen_q < 0 || max_seqlen_q > total_q) return GQA_ERR_INVALID_ARG;
  if (max_kv_len < 1 || max_kv_len > kv_cap) return GQA_ERR_INVALID_ARG;
  if (H_q % H_kv != 0) return GQA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16) return GQA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return GQA_ERR_INVALID_ARG;
  if (d != kD || dtype != GQA_DTYPE_BF16) return GQA_ERR_UNSUPPORTED;
  if ((long long)total_q * H_q * kD >= (1LL << 62)) return GQA_ERR_INVALID_ARG;
  if (max_seqlen_q == 0) return GQA_OK;
  const int hpw = gqa::prefill_heads_per_wg(H_q / H_kv);
  const long long rows_per_wg = gqa::prefill_rows_per_wg() / hpw;
  const long long n_qblk = ((long long)max_seqlen_q + rows_per_wg - 1) / rows_per_wg;
  if (n_qblk * B * H_kv * ((H_q / H_kv) / hpw) > 0x7fffffffLL) return GQA_ERR_INVALID_ARG;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) ||
      workspace_bytes < gqa::prefill_varlen_sched_bytes(B, n_qblk))
    return GQA_ERR_WORKSPACE;

  gqa::PrefillParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.H_q = H_q;
  p.H_kv = H_kv;
  p.G = H_q / H_kv;
  p.S_q = total_q;
  p.S_kv = max_kv_len;
  p.kv_cap = kv_cap;
  p.causal = causal;
  p.offset = 0;
  p.heads_per_wg = hpw;
  p.n_qblk = (int)n_qblk;
  p.q_negate = scale < 0.f;
  p.pair_blocks = 0;
  p.scale_log2 = fabsf(scale) * 1.4426950408889634f;
  p.cu_seqlens_q = cu_seqlens_q;
  p.kv_lens = kv_lens;
  p.sched = static_cast<int*>(workspace);
  p.block_table = block_table;
  p.max_pages = max_pages;
  p.page_shift = page_shift;
  p.num_pages = num_pages;
  hipError_t e = gqa::launch_prefill(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int gqa_attn_prefill_varlen(const void* q, const void* k, const void* v, const int* cu_seqlens_q,
                            const int* kv_lens, void* o, float* lse, int B, int H_q, int H_kv,
                            int d, int total_q, int max_seqlen_q, int kv_cap, int max_kv_len,
                            int causal, float scale, int dtype, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return prefill_varlen_common(q, k, v, cu_seqlens_q, kv_lens, o, lse, B, H_q, H_kv, d, total_q,
                               max_seqlen_q, kv_cap, max_kv_len, causal, scale, dtype, workspace,
                               workspace_bytes, stream, nullptr, 0, 0, 0);
}

int gqa_attn_prefill_paged(const void* q, const void* k_pages, const void* v_pages,
                           const int* block_table, const int* cu_seqlens_q, const int* kv_lens,
                           void* o, float* lse, int B, int H_q, int H_kv, int d, int total_q,
                           int max_seqlen_q, int page_size, int max_pages_per_seq, int num_pages,
                           int max_kv_len, int causal, float scale, int dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!block_table || (reinterpret_cast<uintptr_t>(block_table) & 3u)) return GQA_ERR_INVALID_ARG;
  const int sh = page_shift_of(page_size);
  if (sh < 0 || max_pages_per_seq < 1 || num_pages < 1) return GQA_ERR_INVALID_ARG;
  if (H_kv >= 1 && (long long)num_pages * H_kv * page_size * kD >= (1LL << 62))
    return GQA_ERR_INVALID_ARG;
  const long long cap = (long long)max_pages_per_seq * page_size;
  if (max_kv_len < 1 || max_kv_len > cap) return GQA_ERR_INVALID_ARG;
  if ((long long)B * max_pages_per_seq >= (1LL << 31)) return GQA_ERR_INVALID_ARG;
  // The kernel stages one table row in LDS: at most kPrefillMaxPages pages
  // of a sequence are reachable.
  if (((long long)max_kv_len + page_size - 1) / page_size > gqa::kPrefillMaxPages)
    return GQA_ERR_UNSUPPORTED;
  return prefill_varlen_common(q, k_pages, v_pages, cu_seqlens_q, kv_lens, o, lse, B, H_q, H_kv,
                               d, total_q, max_seqlen_q, (int)(cap < 0x7fffffff ? cap : 0x7fffffff),
                               max_kv_len, causal, scale, dtype, workspace, workspace_bytes,
                               stream, block_table, sh, max_pages_per_seq, num_pages);
}

}  // extern "C"
