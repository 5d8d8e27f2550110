// Causal (or full) prefill attention for gfx950.
//
// Method: ADR-0060 "AHBM GQA Fused Attention Kernel (Llama3-70B)", revision
// 5a76ed4 -- §3 (per-tile op sequence: scores, optional mask on boundary
// tiles, online softmax, fused P.V, one normalisation at the end), §5.4
// (causal tile classes: tiles wholly before the query block run unmasked,
// tiles wholly after it are skipped, only the diagonal tile is masked; the
// group's query heads are batched along the same axis as in decode),
// §0.5.3 (q_block_meta: the chunk follows `offset` cached tokens) and §5.6
// option 3 (issue the next tile's Q.K^T before the current softmax so the
// matrix unit is not idle while the softmax runs).
//
// GPU mapping.  One workgroup = 8 waves (two per SIMD) = 256 query rows that
// share one KV head: with G = 8 each wave is one query head of the group over
// the same 32 positions (the pages' M-fold), so every K/V tile staged in LDS
// serves 256 rows and all waves share one causal extent.  In general the 8
// waves cover gcd(G, 8) heads x 8/gcd(G, 8) consecutive 32-position blocks.
//
// Per wave and 64-key tile: S^T = K . Q^T on the 32x32x16 bf16 MFMA (keys in
// M, the wave's 32 queries in N, Q held in registers), so each lane owns 32
// of its query's 64 scores (the other 32 sit in lane ^ 32); P is rounded to
// bf16 in registers and is directly the B operand of O^T = V^T . P^T, whose
// V^T operand comes from the row-major V tile through the gfx950 LDS
// transpose read (ds_read_b64_tr_b16).
//
// Tiles reach LDS with direct global->LDS loads (no staging registers),
// XOR-swizzled per 16-byte piece so that both the K operand reads and the
// V transpose reads are bank-conflict free.  K and V are triple-buffered:
// step j issues S of tile j+1 and P.V of tile j-1 (32 MFMAs) next to the
// softmax of tile j, one straight-line block per step.
//
// Softmax in the log2 domain with a lazy per-row reference max: exps use
// the reference r, p = exp2(s*scale - r); the reference moves only when a
// tile's max exceeds r + 64 (then r = max - 32, and O and l are rescaled),
// which in practice happens on the first tile only.  O and l share the
// reference, so O / l and the LSE are exact.  The common step therefore
// needs no cross-lane exchange: each lane tests its own 32 scores and a
// wave vote sends the rare case to a fix-up path that recomputes the tile.
// Row sums are accumulated in fp32 from the unrounded P, so the exported
// LSE carries no bf16 rounding.
//
// Workgroup order: the KV head is the fastest-varying index, so with the
// round-robin dispatch of workgroups over the 8 XCDs each KV head's tiles
// stay in one XCD's L2; query blocks go heaviest (longest causal prefix)
// first.

#include "common.hpp"
#include "kernels.hpp"

namespace gqa {

namespace {

constexpr int kD = 128;
constexpr int kBN = 64;              // keys per tile
constexpr int kWaves = 8;            // waves per workgroup: two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kTileElems = kBN * kD; // 16 KiB of bf16 per tile, unpadded
constexpr int kBufs = 3;
constexpr float kResetGap = 64.f;    // log2 units
constexpr float kRefBelow = 32.f;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ s16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Physical 16-byte piece of logical piece `pc` (0..15) in tile row `row`.
__device__ __forceinline__ int k_swz(int row, int pc) { return pc ^ (row & 15); }
__device__ __forceinline__ int v_swz(int row, int pc) { return pc ^ ((row & 3) << 2); }

struct Tile16 {
  f32x16 s[2];   // S^T of keys kbase + 32*mt + 8*(i/4) + 4*h2 + (i%4), query c
};

struct PTile {
  bf16x8 p[4];   // P of 16-key step st: keys 16*st + {0..3, 8..11} + 4*h2, query c
};

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) __bf16 sK[kBufs][kTileElems];
  __shared__ __attribute__((aligned(1024))) __bf16 sV[kBufs][kTileElems];

  // Workgroup -> (position block, sequence, head group, KV head).
  const int hpw = p.heads_per_wg;
  const int pbw = kWaves / hpw;          // 32-position blocks per workgroup
  const int ngroups = p.G / hpw;
  int id = blockIdx.x;
  const int kvh = id % p.H_kv;
  id /= p.H_kv;
  const int hg = id % ngroups;
  id /= ngroups;
  const int b = id % p.B;
  id /= p.B;
  const int pblk = p.n_qblk - 1 - id;

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int c = lane & 31;       // query column of this lane
  const int h2 = lane >> 5;      // half of the wave
  const int t16 = lane & 15;
  const int gamma = lane >> 4;

  const int h = kvh * p.G + hg * hpw + wave % hpw;
  const int P0 = pblk * 32 * pbw;
  const int qw0 = P0 + 32 * (wave / hpw);   // first row of this wave
  const int qrow = qw0 + c;                 // this lane's query row

  int kend = p.S_kv;
  if (p.causal) kend = min(kend, p.offset + P0 + 32 * pbw);
  const int ntiles = (kend + kBN - 1) / kBN;
  // Tiles [0, n_full) need no mask for this wave, [n_full, n_live) are
  // masked (diagonal or past S_kv), the rest are invisible to all its rows.
  int n_live = ntiles;
  int n_full = p.S_kv / kBN;
  if (p.causal) {
    n_live = min(ntiles, (p.offset + qw0 + 31) / kBN + 1);
    n_full = min(n_full, (p.offset + qw0 + 1) / kBN);
  }
  n_full = min(n_full, n_live);

  const __bf16* Q = static_cast<const __bf16*>(p.q) + ((size_t)b * p.H_q + h) * p.S_q * kD;
  const __bf16* Kg = static_cast<const __bf16*>(p.k) + ((size_t)b * p.H_kv + kvh) * p.kv_cap * kD;
  const __bf16* Vg = static_cast<const __bf16*>(p.v) + ((size_t)b * p.H_kv + kvh) * p.kv_cap * kD;

  // Q^T operand (B of S^T): query qrow, d = 16*ks + 8*h2 .. +8.  A negative
  // scale is applied exactly by flipping Q's sign bits.
  bf16x8 qb[8];
  {
    const bool ok = qrow < p.S_q;
    const __bf16* qr = Q + (size_t)(ok ? qrow : 0) * kD + 8 * h2;
    const unsigned flip = p.q_negate ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 v = ok ? ld16(qr + 16 * ks) : u32x4{0, 0, 0, 0};
      v ^= u32x4{flip, flip, flip, flip};
      qb[ks] = as_bf16x8(v);
    }
  }

  // Direct global -> LDS tile load: the waves split the 16 row groups of 4
  // rows; one 1 KiB instruction fills a group, lane l landing at physical
  // piece l%16 of row 4*group + l/16 and fetching the logical piece that
  // belongs there.  Rows
  // past S_kv re-read the last valid row (finite data; those keys are
  // masked and their V rows get weight 0).
  auto tile_load = [&](__bf16* buf, const __bf16* g, int tile, bool is_v) {
    constexpr int kInsts = kBN / 4 / kWaves;   // 1 KiB (4-row) loads per wave
#pragma unroll
    for (int i = 0; i < kInsts; ++i) {
      const int row0 = 4 * (kInsts * wave + i);
      const int row = row0 + (lane >> 4);
      const int phys = lane & 15;
      const int logical = is_v ? v_swz(row, phys) : k_swz(row, phys);   // XOR is an involution
      const int key = min(tile * kBN + row, p.S_kv - 1);
      const __bf16* src = g + (size_t)key * kD + logical * 8;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(buf + row0 * kD), 16, 0, 0);
    }
  };

  // S^T of one tile from K buffer `kb`.
  auto compute_s = [&](Tile16& T, const __bf16* kb) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int row = 32 * mt + c;
      const __bf16* kr = kb + row * kD;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + 8 * k_swz(row, 2 * ks + h2));
        const f32x16 zero = {};
        T.s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], ks ? T.s[mt] : zero, 0, 0, 0);
      }
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

  // O^T += V^T . P^T for one tile from V buffer `vb`.  Lane (gamma, t16)
  // supplies the address of row r0 + t16/4, d = 32*dt + 16*(gamma&1) +
  // 4*(t16&3) .. +4, and receives V^T column d = 32*dt + 16*(gamma&1) + t16.
  auto pv = [&](const PTile& P, const __bf16* vb) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int r0 = 16 * st + 4 * h2 + (t16 >> 2);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int e = 32 * dt + 16 * (gamma & 1) + 4 * (t16 & 3);   // element within the row
        const int pc = e >> 3;
        const int off = e & 7;
        const s16x4 x0 = lds_read_tr16(vb + r0 * kD + 8 * v_swz(r0, pc) + off);
        const s16x4 x1 = lds_read_tr16(vb + (r0 + 8) * kD + 8 * v_swz(r0 + 8, pc) + off);
        u32x4 av;
        av[0] = __builtin_bit_cast(u32x2, x0)[0];
        av[1] = __builtin_bit_cast(u32x2, x0)[1];
        av[2] = __builtin_bit_cast(u32x2, x1)[0];
        av[3] = __builtin_bit_cast(u32x2, x1)[1];
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), P.p[st], o[dt], 0, 0, 0);
      }
    }
  };

  float m_ref = kNegInf;  // reference max (log2 domain) of row qrow, same on both halves
  float lpart = 0.f;      // this lane's half of the running sum
  const float sl2 = p.scale_log2;
  const int vis_last = p.causal ? p.offset + qrow : p.S_kv - 1;

  // P = exp2(S*scale - ref) rounded to bf16; returns the fp32 sum of P over
  // this lane's 32 keys.  Masked scores hold -inf and get weight 0.
  auto exps = [&](const Tile16& T, PTile& P, float ref, bool masked) -> float {
    const float negr = -ref;
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int mt = st >> 1;
      const int sp = st & 1;
      u32x4 pw;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float x0 = T.s[mt][8 * sp + 2 * jj];
        const float x1 = T.s[mt][8 * sp + 2 * jj + 1];
        float e0 = fast_exp2(__builtin_fmaf(x0, sl2, negr));
        float e1 = fast_exp2(__builtin_fmaf(x1, sl2, negr));
        if (masked) {
          e0 = x0 == kNegInf ? 0.f : e0;
          e1 = x1 == kNegInf ? 0.f : e1;
        }
        pw[jj] = pack_bf16x2(e0, e1);
        psum += e0 + e1;
      }
      P.p[st] = as_bf16x8(pw);
    }
    return psum;
  };

  auto mask_tile = [&](Tile16& T, int tile) {
    const int kbase = tile * kBN;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kbase + 32 * mt + 8 * (i >> 2) + 4 * h2 + (i & 3);
        if (key > vis_last || key >= p.S_kv) T.s[mt][i] = kNegInf;
      }
  };

  auto lane_max = [&](const Tile16& T) {
    float r = kNegInf;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) r = fmaxf(r, T.s[mt][i]);
    return r;
  };

  // Softmax of one tile.  The common case keeps the reference; the rare
  // case (first tile, or a jump of the max) moves it with a full row max,
  // rescales O and l, and recomputes P.
  auto softmax = [&](Tile16& T, PTile& P, int tile, bool masked) {
    if (masked) mask_tile(T, tile);
    const float hmax = lane_max(T);
    float psum = exps(T, P, m_ref, masked);
    // Keep the speculative P in this block (next to the step's MFMAs)
    // instead of letting the compiler sink it past the rare branch.
#pragma unroll
    for (int st = 0; st < 4; ++st) asm volatile("" ::"v"(P.p[st]));
    asm volatile("" ::"v"(psum));
    const float hscaled = hmax == kNegInf ? kNegInf : hmax * sl2;
    if (__any(hscaled > m_ref + kResetGap)) {
      const float rmax = wave_max_xor(hscaled, 32);
      const float m_new = rmax > m_ref + kResetGap ? rmax - kRefBelow : m_ref;
      const float corr = fast_exp2(m_ref - m_new);
      lpart *= corr;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= corr;
      m_ref = m_new;
      psum = exps(T, P, m_ref, masked);
    }
    lpart += psum;
  };

  // Prologue: K tiles 0 and 1, V tile 0 in LDS; S of tile 0.
  tile_load(sK[0], Kg, 0, false);
  tile_load(sV[0], Vg, 0, true);
  if (ntiles > 1) tile_load(sK[1], Kg, 1, false);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's tile loads landed
  __syncthreads();
  Tile16 TA, TB;
  PTile PA, PB;
  compute_s(TA, sK[0]);

  // Step j: S of tile j+1 into `nxt`, P.V of tile j-1 from `pprev`, softmax
  // of tile j (scores in `cur`) into `pcur`; K for j+2 and V for j+1 are
  // loaded into the free LDS buffers.
  auto step = [&](Tile16& cur, Tile16& nxt, PTile& pcur, const PTile& pprev, int j) {
    if (j + 2 < ntiles) tile_load(sK[(j + 2) % kBufs], Kg, j + 2, false);
    if (j + 1 < ntiles) tile_load(sV[(j + 1) % kBufs], Vg, j + 1, true);
    const bool do_s = j + 1 < n_live;
    const bool do_pv = j >= 1 && j - 1 < n_live;
    const bool do_sm = j < n_live;
    if (do_s && do_pv && do_sm && j < n_full) {
      compute_s(nxt, sK[(j + 1) % kBufs]);
      pv(pprev, sV[(j - 1) % kBufs]);
      softmax(cur, pcur, j, false);
    } else {
      if (do_s) compute_s(nxt, sK[(j + 1) % kBufs]);
      if (do_pv) pv(pprev, sV[(j - 1) % kBufs]);
      if (do_sm) softmax(cur, pcur, j, j >= n_full);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    step(TA, TB, PA, PB, j);
    step(TB, TA, PB, PA, j + 1);
  }
  if (j < ntiles) {
    step(TA, TB, PA, PB, j);
    if (n_live == ntiles) pv(PA, sV[j % kBufs]);   // P.V of the last tile
  } else if (n_live == ntiles) {
    pv(PB, sV[(j - 1) % kBufs]);
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
      p.lse[((size_t)b * p.H_q + h) * p.S_q + qrow] = (m_ref + __log2f(lsum)) * kLn2;
  }
}

int prefill_heads_per_wg(int G) {
  int a = G, b = kWaves;
  while (b) {
    const int r = a % b;
    a = b;
    b = r;
  }
  return a;   // gcd(G, waves per workgroup)
}

int prefill_rows_per_wg() { return 32 * kWaves; }

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  const long long nwg = (long long)p.n_qblk * p.B * p.H_kv * (p.G / p.heads_per_wg);
  hipLaunchKernelGGL(prefill_bf16_kernel, dim3((unsigned)nwg), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
