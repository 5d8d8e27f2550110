// K/V tiles in LDS for the gfx950 kernels that share one tile between
// several waves: 256-byte bf16 rows (d = 128), XOR-swizzled per 16-byte
// piece, filled by direct global -> LDS loads.
#pragma once

#include "common.hpp"

namespace gqa {

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 32-bit LDS address of a shared-memory object, and back.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(3))) T* lds_ptr(unsigned a) {
  return (const __attribute__((address_space(3))) T*)(uintptr_t)a;
}

// ds_read_b64_tr_b16: each lane receives four 16-bit elements of one column
// of a 4x16 block (the transposing LDS read of gfx950).
__device__ __forceinline__ s16x4 lds_read_tr16(unsigned a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)a);
}

// Physical 16-byte piece of logical piece `pc` (0..15) in tile row `row`.
// K rows: a wave reading one logical piece of 16 consecutive rows touches
// 16 distinct pieces.  V rows: the transposing reads of 4 consecutive rows
// at one d range hit distinct banks.
__device__ __forceinline__ int k_swz(int row, int pc) { return pc ^ (row & 15); }
__device__ __forceinline__ int v_swz(int row, int pc) { return pc ^ ((row & 3) << 2); }

// Buffer resource over `bytes` bytes from `base` (raw buffer, 32-bit data
// format, no stride): reads at or past `bytes` return zeros and touch no
// memory.  The values are made wave-uniform for the scalar operands.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, unsigned bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}

// One 1 KiB direct global -> LDS load: lane l fetches 16 bytes at byte
// offset `voff` of the resource and writes them to LDS address
// `lds_dst + 16*l` (`lds_dst` is wave-uniform).  Issued as inline assembly
// so that the compiler does not make later LDS reads wait for it (it cannot
// tell the addresses apart); the caller waits with s_waitcnt vmcnt before
// the data is read.  Wait states inside the statement: the descriptor and
// M0 value come from v_readfirstlane, and an LDS DMA may not directly
// follow an M0 write.  M0 is a register the compiler reserves: it may
// not be named as clobbered (that is undefined), and the compiler sets it
// immediately before each of its own uses; a CPU test checks that the
// built kernels write and read M0 nowhere but in these sequences.
__device__ __forceinline__ void dma_load_x4(int voff, u32x4 rsrc, unsigned lds_dst) {
  const unsigned dst = __builtin_amdgcn_readfirstlane(lds_dst);
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(dst)
               : "memory");
}


}  // namespace gqa
