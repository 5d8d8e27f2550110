// Shared device helpers for the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Hardware base-2 exponential (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One 16-byte global load (global_load_dwordx4).
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Streaming 16-byte load for data read exactly once (non-temporal hint).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two floats -> two bf16 (round to nearest even) packed in one dword.
__device__ __forceinline__ unsigned int pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(unsigned int, b);
}

// s_waitcnt immediate that waits until at most `n` (0..63) vector memory
// operations of this wave are outstanding (lgkm and exp counters ignored).
constexpr unsigned vmcnt_imm(int n) {
  return 0x0F70u | ((unsigned)n & 15u) | (((unsigned)n >> 4) << 14);
}

__device__ __forceinline__ float wave_max_xor(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask, 64));
}

__device__ __forceinline__ float wave_sum_xor(float x, int mask) {
  return x + __shfl_xor(x, mask, 64);
}

}  // namespace gqa
