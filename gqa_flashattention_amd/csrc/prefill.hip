// Causal (or full) prefill attention for gfx950.
//
// Method: ADR-0060 "AHBM GQA Fused Attention Kernel (Llama3-70B)", revision
// 5a76ed4 -- §3 (per-tile op sequence: scores, optional additive mask on
// boundary tiles, online softmax, fused P.V, one normalisation at the end),
// §5.4 (causal tile classes: tiles wholly before the query block run
// unmasked, tiles wholly after it are skipped, only the diagonal is masked)
// and §0.5.3 (q_block_meta: the chunk follows `offset` cached tokens).
//
// GPU mapping.  One workgroup = 4 waves = 128 query rows of one query head;
// wave w owns rows 32w .. 32w+31.  K/V tiles of 64 keys are staged through
// LDS (double-buffered, one barrier per tile) and shared by the 4 waves.
// S^T = K . Q^T runs on the 32x32x16 bf16 MFMA with keys in M and queries in
// N, so each lane holds one query's 32 scores of a tile and the row max needs
// a single cross-lane step.  P never leaves registers: the S^T accumulator
// layout is already the B operand of O^T = V^T . P^T once rounded to bf16.
// V^T comes straight from the row-major V tile through the gfx950 LDS
// transpose read (ds_read_b64_tr_b16).  The online softmax runs in the log2
// domain; the O rescale is skipped when no row's max moved.
//
// Workgroup order: the fastest-varying index is the KV head, so with the
// round-robin dispatch of workgroups over the 8 XCDs all query heads of one
// KV head land on one XCD and share its L2; query blocks are issued heaviest
// (latest, longest causal prefix) first.

#include "common.hpp"
#include "kernels.hpp"

namespace gqa {

namespace {

constexpr int kD = 128;
constexpr int kBM = kPrefillBlockM;  // 128 query rows per workgroup
constexpr int kBN = 64;              // keys per tile
constexpr int kKStride = kD + 8;     // LDS row pitch of K (bf16 elements)
constexpr int kVStride = kD + 16;    // LDS row pitch of V (bf16 elements)

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ s16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

}  // namespace

__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 sK[2][kBN * kKStride];
  __shared__ __attribute__((aligned(16))) __bf16 sV[2][kBN * kVStride];

  // Workgroup -> (query block, sequence, query head).
  int w = blockIdx.x;
  const int kvh = w % p.H_kv;
  w /= p.H_kv;
  const int gq = w % p.G;
  w /= p.G;
  const int b = w % p.B;
  w /= p.B;
  const int qblk = p.n_qblk - 1 - w;
  const int h = kvh * p.G + gq;
  const int q0 = qblk * kBM;

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int c = lane & 31;       // query column of this lane
  const int h2 = lane >> 5;      // which half of the wave
  const int t16 = lane & 15;
  const int gamma = lane >> 4;

  const int qw0 = q0 + 32 * wave;   // first row of this wave
  const int qrow = qw0 + c;         // this lane's query row

  int kend = p.S_kv;
  if (p.causal) kend = min(kend, p.offset + q0 + kBM);
  const int ntiles = (kend + kBN - 1) / kBN;

  const __bf16* Q = static_cast<const __bf16*>(p.q) + ((size_t)b * p.H_q + h) * p.S_q * kD;
  const __bf16* Kg = static_cast<const __bf16*>(p.k) + ((size_t)b * p.H_kv + kvh) * p.kv_cap * kD;
  const __bf16* Vg = static_cast<const __bf16*>(p.v) + ((size_t)b * p.H_kv + kvh) * p.kv_cap * kD;

  // Q^T operand (B of S^T): query qrow, d = 16*ks + 8*h2 .. +8.
  bf16x8 qb[8];
  {
    const bool ok = qrow < p.S_q;
    const __bf16* qr = Q + (size_t)(ok ? qrow : 0) * kD + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qb[ks] = as_bf16x8(ok ? ld16(qr + 16 * ks) : u32x4{0, 0, 0, 0});
  }

  // Global -> register staging: thread t moves 16-byte pieces t + 256*r of
  // the 64x128 K and V tiles (row = piece / 16, column = 8 * (piece % 16)).
  u32x4 kst[4], vst[4];
  auto gload = [&](int tile) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int idx = t + 256 * r;
      const int key = tile * kBN + (idx >> 4);
      const int col = (idx & 15) * 8;
      const bool ok = key < p.S_kv;
      kst[r] = ok ? ld16(Kg + (size_t)key * kD + col) : u32x4{0, 0, 0, 0};
      vst[r] = ok ? ld16(Vg + (size_t)key * kD + col) : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int idx = t + 256 * r;
      const int row = idx >> 4;
      const int col = (idx & 15) * 8;
      *reinterpret_cast<u32x4*>(&sK[buf][row * kKStride + col]) = kst[r];
      *reinterpret_cast<u32x4*>(&sV[buf][row * kVStride + col]) = vst[r];
    }
  };

  float m = kNegInf;    // running max (log2 domain) of row qrow
  float lpart = 0.f;    // this lane's half of the running sum
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ntiles) gload(kt + 1);

    const int kbase = kt * kBN;
    const bool wave_live = !p.causal || kbase <= p.offset + qw0 + 31;
    if (wave_live) {
      const bool need_mask = (p.causal && kbase + kBN - 1 > p.offset + qw0) || kbase + kBN > p.S_kv;
      // S^T for keys kbase + 32*mt + (0..31).
      f32x16 s[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[mt][i] = 0.f;
        const __bf16* kr = &sK[buf][(32 * mt + c) * kKStride + 8 * h2];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + 16 * ks);
          s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], s[mt], 0, 0, 0);
        }
      }
      // Scale, mask, row max.  Element i of tile mt is key
      // kbase + 32*mt + 8*(i/4) + 4*h2 + (i%4).
      float tmax = kNegInf;
      const int vis_last = p.causal ? p.offset + qrow : p.S_kv - 1;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = s[mt][i] * p.scale_log2;
          if (need_mask) {
            const int key = kbase + 32 * mt + 8 * (i >> 2) + 4 * h2 + (i & 3);
            if (key > vis_last || key >= p.S_kv) x = kNegInf;
          }
          s[mt][i] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = wave_max_xor(tmax, 32);
      const float m_new = fmaxf(m, tmax);
      const float corr = fast_exp2(m - m_new);
      float psum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = fast_exp2(s[mt][i] - m_new);
          s[mt][i] = e;
          psum += e;
        }
      lpart = lpart * corr + psum;
      if (__any(m_new > m)) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] *= corr;
      }
      m = m_new;

      // O^T += V^T . P^T in four 16-key steps.
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int mt = st >> 1;
        const int sp = st & 1;
        u32x4 pw;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          pw[jj] = pack_bf16x2(s[mt][8 * sp + 2 * jj], s[mt][8 * sp + 2 * jj + 1]);
        const bf16x8 pb = as_bf16x8(pw);
        const int r0 = 32 * mt + 16 * sp + 4 * h2 + (t16 >> 2);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int col = 32 * dt + 16 * (gamma & 1) + 4 * (t16 & 3);
          const s16x4 x0 = lds_read_tr16(&sV[buf][r0 * kVStride + col]);
          const s16x4 x1 = lds_read_tr16(&sV[buf][(r0 + 8) * kVStride + col]);
          u32x4 av;
          av[0] = __builtin_bit_cast(u32x2, x0)[0];
          av[1] = __builtin_bit_cast(u32x2, x0)[1];
          av[2] = __builtin_bit_cast(u32x2, x1)[0];
          av[3] = __builtin_bit_cast(u32x2, x1)[1];
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), pb, o[dt], 0, 0, 0);
        }
      }
    }

    if (kt + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: O = O / l, rounded to bf16.  Lane holds, for d-tile dt and
  // i = 0..15, d = 32*dt + 8*(i/4) + 4*h2 + (i%4) of row qrow.
  const float lsum = lpart + __shfl_xor(lpart, 32, 64);
  if (qrow < p.S_q) {
    const float inv = 1.f / lsum;
    __bf16* orow = static_cast<__bf16*>(p.o) + (((size_t)b * p.H_q + h) * p.S_q + qrow) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = 32 * dt + 8 * i4 + 4 * h2;
        u32x2 v2 = {pack_bf16x2(o[dt][4 * i4] * inv, o[dt][4 * i4 + 1] * inv),
                    pack_bf16x2(o[dt][4 * i4 + 2] * inv, o[dt][4 * i4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = v2;
      }
    if (p.lse != nullptr && h2 == 0)
      p.lse[((size_t)b * p.H_q + h) * p.S_q + qrow] = (m + __log2f(lsum)) * kLn2;
  }
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  const long long nwg = (long long)p.n_qblk * p.B * p.H_q;
  hipLaunchKernelGGL(prefill_bf16_kernel, dim3((unsigned)nwg), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
