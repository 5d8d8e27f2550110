// Stitching of two attention results over disjoint key sets (chunked
// prefill against a cached prefix, KV split across calls or devices): the
// log-sum-exp merge of ADR-0060 "AHBM GQA Fused Attention Kernel
// (Llama3-70B)", revision 5a76ed4, §4, applied to normalised results.
//
// A normalised result (O, lse) is the partial (m, l, O) = (lse, 1, O), so
// the merge is M = max(lse_a, lse_b), w = exp(lse - M) per side,
// O = (w_a O_a + w_b O_b) / (w_a + w_b), lse = M + ln(w_a + w_b).  A side
// with lse = -inf (no visible key) has weight 0 and its O is not read into
// the sum (it may be anything, NaN included).
//
// GPU mapping: 16 lanes per row of d = 128, 8 elements (16 bytes of bf16,
// 32 of fp32) per lane; a row never spans two waves, so the output may
// alias either input (each lane reads its elements and the row's LSEs
// before any lane of the wave writes).  HBM bound: 3 rows of O and 3 LSEs
// per row.

#include "common.hpp"
#include "kernels.hpp"

namespace gqa {

namespace {

constexpr int kD = 128;
constexpr int kLanesPerRow = kD / 8;
constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kLanesPerRow;

__device__ __forceinline__ void load8(const __bf16* p, float (&x)[8]) {
  const u32x4 v = ld16_stream(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(v[i] << 16);
    x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}
__device__ __forceinline__ void store8(__bf16* p, const float (&x)[8]) {
  const u32x4 v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7])};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(p));
  __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, reinterpret_cast<f32x4*>(p) + 1);
}

}  // namespace

template <typename T>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeParams p) {
  const long long row = (long long)blockIdx.x * kRowsPerBlock + (threadIdx.x / kLanesPerRow);
  if (row >= p.rows) return;
  const int c0 = (threadIdx.x % kLanesPerRow) * 8;
  const T* oa = static_cast<const T*>(p.o_a) + row * kD + c0;
  const T* ob = static_cast<const T*>(p.o_b) + row * kD + c0;
  const float la = p.lse_a[row];
  const float lb = p.lse_b[row];
  float xa[8], xb[8];
  load8(oa, xa);
  load8(ob, xb);
  const float M = fmaxf(la, lb);
  // Weights exp(lse - M) in base 2; an empty side (-inf) has weight 0 and
  // is selected away, not multiplied.  With both sides empty, M = -inf:
  // the output is O = 0, lse = -inf.
  const bool ea = la == kNegInf, eb = lb == kNegInf;
  const float ref = M == kNegInf ? 0.f : M;
  const float wa = ea ? 0.f : fast_exp2((la - ref) * kLog2e);
  const float wb = eb ? 0.f : fast_exp2((lb - ref) * kLog2e);
  const float wsum = wa + wb;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float ta = ea ? 0.f : wa * xa[i];
    const float tb = eb ? 0.f : wb * xb[i];
    y[i] = (ta + tb) * inv;
  }
  store8(static_cast<T*>(p.o_out) + row * kD + c0, y);
  if (p.lse_out != nullptr && c0 == 0)
    p.lse_out[row] = wsum > 0.f ? M + __log2f(wsum) * kLn2 : kNegInf;
}

hipError_t launch_merge(const MergeParams& p, bool bf16, hipStream_t stream) {
  const long long blocks = (p.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (bf16) {
    hipLaunchKernelGGL(merge_kernel<__bf16>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(merge_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace gqa
