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
// V transpose reads are bank-conflict free.  K and V sit in 4-deep rings:
// step j issues P.V of tile j-1 and S of tile j+1 (32 MFMAs) with the
// softmax of tile j spread between them, one straight-line block per step.
//
// Softmax in the log2 domain with a lazy per-row reference max: exps use
// the reference r, p = exp2(s*scale - r); the reference moves only when a
// tile's max exceeds r + 64 (then r = max - 32, and O and l are rescaled);
// the prologue sets r from tile 0, so in practice it never moves.  O and
// l share the reference, so O / l and the LSE are exact.  The common step
// therefore needs no cross-lane exchange: each lane tests its own 32
// scores and a wave vote sends the rare case to a fix-up path that
// recomputes the tile.
// Row sums are accumulated in fp32 from the unrounded P, so the exported
// LSE carries no bf16 rounding.
//
// Workgroup order: the KV head is the fastest-varying index, so with the
// round-robin dispatch of workgroups over the 8 XCDs each KV head's tiles
// stay in one XCD's L2; query blocks go heaviest (longest causal prefix)
// first.  A causal dense launch pairs each block with its mirror in one
// workgroup (the heaviest with the lightest, and so on): every workgroup
// then does about the same work, and half as many workgroups start.
//
// Varlen batches (chunks of several sequences in one launch, each the newest
// positions of its sequence): the same kernel, with each workgroup reading
// its sequence's chunk length and key count and taking the causal offset
// (keys) - (chunk length), q_block_meta of §0.5.3 per sequence.  The
// lengths live on the device, so a one-workgroup pre-pass sorts the
// (sequence, position block) items by their tile count (a counting sort in
// LDS) into a work list, heaviest first, and workgroup i takes item i: a
// long chunk over a long cache starts first instead of trailing the grid.
// Items past a chunk's end cost nothing and sort last.

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_tile.hpp"

namespace gqa {

namespace {

constexpr int kD = 128;
constexpr int kBN = 64;              // keys per tile
constexpr int kWaves = 8;            // waves per workgroup: two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kTileElems = kBN * kD; // 16 KiB of bf16 per tile, unpadded
constexpr int kBufs = 4;              // K and V tile rings (tile t in buffer t % 4)

constexpr float kResetGap = 64.f;    // log2 units
constexpr float kPsumLimit = 18446744073709551616.f;   // 2^64 = exp2(kResetGap)
constexpr float kRefBelow = 32.f;

constexpr int kTileBytes = kTileElems * 2;

struct Tile16 {
  f32x16 s[2];   // S^T of keys kbase + 32*mt + 8*(i/4) + 4*h2 + (i%4), query c
};

struct PTile {
  bf16x8 p[4];   // P of 16-key step st: keys 16*st + {0..3, 8..11} + 4*h2, query c
};

template <int N>
using Int = std::integral_constant<int, N>;

}  // namespace

// kVarlen: a batch of chunks of different lengths, token-packed.  Sequence
// b's chunk is q/o rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of
// [total_q, H_q, d] (lse [total_q, H_q]) against kv_lens[b] cached keys,
// with causal offset kv_lens[b] - S_q_b; otherwise q/o are [B, H_q, S_q, d].
// kPaged (with kVarlen): K/V come from page pools through the block table.
template <bool kVarlen, bool kPaged>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(PrefillParams p) {
  static_assert(kVarlen || !kPaged, "the paged form is a varlen batch");
  __shared__ __attribute__((aligned(1024))) __bf16 sK[kBufs][kTileElems];
  // Paged form: this sequence's block-table row, clamped into the pool
  // (the 32 KiB the tile rings leave free).
  __shared__ int sPage[kPaged ? kPrefillMaxPages : 1];
  __shared__ __attribute__((aligned(1024))) __bf16 sV[kBufs][kTileElems];

  // Workgroup and wave -> (sequence, position block, query head, KV head),
  // this sequence's chunk length, key count and causal offset, and the
  // addressing of the wave's query rows: row i of head h is row
  // `qrow0 + i * qstride` of the [rows, d] view of q, o and lse.  Varlen
  // sizes come from device arrays and are clamped, so a malformed array
  // cannot move any access outside the buffers (it only makes the results
  // meaningless).  The epilogue evaluates this again from opaque copies of
  // the ids instead of keeping the results live across the main loop.
  struct Place {
    int b, kvh, h, P0, qw0, S_q, S_kv, offset, qstride;
    size_t qrow0;
  };
  auto locate = [&](const auto& p, int bid, int wave_u) -> Place {
    Place L;
    const int hpw = p.heads_per_wg;
    const int ngroups = p.G / hpw;
    int id = bid;
    L.kvh = id % p.H_kv;
    id /= p.H_kv;
    const int hg = id % ngroups;
    id /= ngroups;
    int pblk;
    if constexpr (kVarlen) {
      // Work-list entry b * n_qblk + pblk, clamped into range.
      const unsigned n_items = (unsigned)p.B * (unsigned)p.n_qblk;
      const unsigned item = min((unsigned)p.sched[id], n_items - 1u);
      L.b = (int)(item / (unsigned)p.n_qblk);
      pblk = (int)(item % (unsigned)p.n_qblk);
    } else {
      L.b = id % p.B;
      id /= p.B;
      pblk = p.n_qblk - 1 - id;
    }
    L.h = L.kvh * p.G + hg * hpw + wave_u % hpw;
    L.P0 = pblk * 32 * (kWaves / hpw);
    L.qw0 = L.P0 + 32 * (wave_u / hpw);   // first row of this wave
    if constexpr (kVarlen) {
      const int t0 = min(max(p.cu_seqlens_q[L.b], 0), p.S_q);
      const int t1 = min(max(p.cu_seqlens_q[L.b + 1], t0), p.S_q);
      L.S_q = t1 - t0;
      L.S_kv = min(max(p.kv_lens[L.b], 0), p.S_kv);
      L.offset = p.causal ? max(L.S_kv - L.S_q, 0) : 0;
      L.qrow0 = (size_t)t0 * p.H_q + L.h;
      L.qstride = p.H_q;
    } else {
      L.S_q = p.S_q;
      L.S_kv = p.S_kv;
      L.offset = p.offset;
      L.qrow0 = ((size_t)L.b * p.H_q + L.h) * p.S_q;
      L.qstride = 1;
    }
    return L;
  };

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int c = lane & 31;       // query column of this lane
  const int h2 = lane >> 5;      // half of the wave
  const int t16 = lane & 15;
  const int gamma = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  // One 32-position block (of each wave's head) from start to end; `vid` is
  // the block's workgroup id in the unpaired grid.  The body is not
  // re-indented inside the lambda.
  auto run_block = [&](const int vid) __attribute__((always_inline)) {
  const Place pl = locate(p, vid, wv);
  const int b = pl.b, kvh = pl.kvh, P0 = pl.P0, qw0 = pl.qw0;
  const int S_q = pl.S_q, S_kv = pl.S_kv, offset = pl.offset, qstride = pl.qstride;
  const size_t qrow0 = pl.qrow0;
  const int pbw = kWaves / p.heads_per_wg;   // 32-position blocks per workgroup
  const int qrow = qw0 + c;                   // this lane's query row

  if (P0 >= S_q) return;   // the whole workgroup: past this chunk's end
  if (kVarlen && S_kv == 0) {
    // No key (an empty sequence, varlen only: the dense launch has
    // S_kv >= 1): O = 0, lse = -inf, the convention for a row that sees
    // nothing.  The rows are addressed from opaque copies of the ids, as in
    // the epilogue: this block is laid out after the main loop, and values
    // shared with the loop's prologue would otherwise stay live across it.
    int tid_z = threadIdx.x, bid_z = vid;
    asm volatile("" : "+v"(tid_z), "+s"(bid_z));
    const Place pz = locate(p, bid_z, __builtin_amdgcn_readfirstlane(tid_z >> 6));
    const int qrow_z = pz.qw0 + (tid_z & 31), h2_z = (tid_z >> 5) & 1;
    if (qrow_z < pz.S_q) {
      __bf16* orow = static_cast<__bf16*>(p.o) + (pz.qrow0 + (size_t)qrow_z * pz.qstride) * kD;
      for (int d0 = 4 * h2_z; d0 < kD; d0 += 8)
        *reinterpret_cast<u32x2*>(orow + d0) = u32x2{0, 0};
      if (p.lse != nullptr && h2_z == 0) p.lse[pz.qrow0 + (size_t)qrow_z * pz.qstride] = kNegInf;
    }
    return;
  }

  int kend = S_kv;
  if (p.causal) kend = min(kend, offset + P0 + 32 * pbw);
  const int ntiles = (kend + kBN - 1) / kBN;
  // Tiles [0, n_full) need no mask for this wave, [n_full, n_live) are
  // masked (diagonal or past S_kv), the rest are invisible to all its rows.
  int n_live = ntiles;
  int n_full = S_kv / kBN;
  if (p.causal) {
    n_live = min(ntiles, (offset + qw0 + 31) / kBN + 1);
    n_full = min(n_full, (offset + qw0 + 1) / kBN);
  }
  n_full = min(n_full, n_live);

  // K/V of this (sequence, KV head); the paged form addresses the pools.
  const size_t kv_base = kPaged ? 0 : ((size_t)b * p.H_kv + kvh) * p.kv_cap * kD;
  const __bf16* Kg = static_cast<const __bf16*>(p.k) + kv_base;
  const __bf16* Vg = static_cast<const __bf16*>(p.v) + kv_base;

  // Q^T operand (B of S^T): query qrow, d = 16*ks + 8*h2 .. +8, through a
  // buffer resource over the wave's rows below S_q, so that rows past the
  // chunk read as zeros without a branch (a branch per load made the
  // compiler wait for the first loads before issuing the rest, and so
  // before the tile loads).  A negative scale is applied exactly by flipping
  // Q's sign bits, in a branch of its own so that the common case does not
  // wait for Q before the tile loads are issued.
  bf16x8 qb[8];
  {
    const int nq = min(max(S_q - qw0, 0), 32);   // the wave's rows inside the chunk
    // Wave-uniform by construction; readfirstlane says so to the compiler,
    // which otherwise loops over the lanes' descriptors.
    const uintptr_t qa =
        reinterpret_cast<uintptr_t>(static_cast<const __bf16*>(p.q) + (qrow0 + (size_t)qw0 * qstride) * kD);
    // (readfirstlane returns an int: each half goes through unsigned so
    // that the low one is not sign-extended into the high one.)
    const uintptr_t qau = ((uintptr_t)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)(qa >> 32)) << 32) |
                          (uintptr_t)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)qa);
    const unsigned bytes = __builtin_amdgcn_readfirstlane(
        nq > 0 ? (unsigned)((nq - 1) * qstride + 1) * (kD * 2) : 0u);
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(qau), (short)0, bytes, 0x00020000);
    const int off = c * qstride * (kD * 2) + 16 * h2;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qb[ks] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rq, off + 32 * ks, 0, 0));
    if (p.q_negate) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        u32x4 v = __builtin_bit_cast(u32x4, qb[ks]);
        v ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        qb[ks] = as_bf16x8(v);
      }
    }
  }

  // Per-lane LDS byte addresses of the MFMA operands in buffer 0; other
  // buffers and sub-blocks are immediate offsets (all below 64 KiB).
  //  K (A of S^T), k-step ks, sub-tile mt: row 32*mt + c, logical piece
  //    2*ks + h2; row + 32 has the same swizzle, so mt adds 8 KiB.
  //  V (A of O^T, transposed read), key step st, d-tile dt: rows
  //    r0 = 16*st + 4*h2 + t16/4 and r0 + 8, element e = 32*dt +
  //    16*(gamma&1) + 4*(t16&3); r0 & 3 does not depend on st, so st adds
  //    4 KiB and the second row 2 KiB.
  // The addresses are hidden from the compiler so that it cannot fold the
  // arrays' base into the 16-bit offsets (which would overflow them).
  unsigned kaddr[8], vaddr[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    kaddr[ks] = lds_addr(&sK[0][0]) + c * 256 + 16 * k_swz(c, 2 * ks + h2);
    asm volatile("" : "+v"(kaddr[ks]));
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int r0 = 4 * h2 + (t16 >> 2);
    const int e = 32 * dt + 16 * (gamma & 1) + 4 * (t16 & 3);
    vaddr[dt] = lds_addr(&sV[0][0]) + r0 * 256 + 16 * v_swz(r0, e >> 3) + 2 * (e & 7);
    asm volatile("" : "+v"(vaddr[dt]));
  }
  auto k_opnd = [&](int buf, int mt, int ks) -> bf16x8 {
    return *lds_ptr<bf16x8>(kaddr[ks] + kTileBytes * buf + 8192 * mt);
  };
  auto v_opnd = [&](int buf, int st, int dt) -> bf16x8 {
    const unsigned a = vaddr[dt] + kTileBytes * buf + 4096 * st;
    const u32x2 w0 = __builtin_bit_cast(u32x2, lds_read_tr16(a));
    const u32x2 w1 = __builtin_bit_cast(u32x2, lds_read_tr16(a + 2048));
    const u32x4 av = {w0[0], w0[1], w1[0], w1[1]};
    return as_bf16x8(av);
  };

  // Direct global -> LDS tile load: the waves split the 16 row groups of 4
  // rows; one 1 KiB instruction fills a group, lane l landing at physical
  // piece l%16 of row 4*group + l/16 and fetching the logical piece that
  // belongs there.  The loads go through a buffer resource that covers only
  // the tile's valid rows (at most 64, below S_kv), so rows past S_kv read
  // as zeros (no clamping, nothing outside the valid rows is touched, and
  // the resource's 32-bit size cannot overflow for any cache length); those
  // keys are masked and their zero V rows get weight 0.  Tile indices past the last tile are clamped to it (the
  // buffers they fill are never read).
  // Paged form: a wave's two instructions cover rows 8w .. 8w+7 of the
  // tile, which lie in one page (pages hold at least 16 rows, a power of
  // two).  The resource is based so that those rows' offsets within the
  // tile land on them in the page, and it ends at the sequence's last key.
  constexpr int kInsts = kBN / 4 / kWaves;   // 1 KiB (4-row) loads per wave
  int ld_off[2][kInsts];                     // [K, V][instruction]: byte offset in a tile
#pragma unroll
  for (int i = 0; i < kInsts; ++i) {
    const int row = 4 * (kInsts * wave + i) + (lane >> 4);
    ld_off[0][i] = row * (kD * 2) + 16 * k_swz(row, lane & 15);   // XOR is an involution
    ld_off[1][i] = row * (kD * 2) + 16 * v_swz(row, lane & 15);
  }
  const unsigned lds_k0 = lds_addr(&sK[0][0]), lds_v0 = lds_addr(&sV[0][0]);
  // One load instruction (i) of tile `tile` of K (kv = 0) or V (kv = 1)
  // into LDS buffer `buf`.  Issued as inline assembly: the compiler would
  // otherwise make the next LDS read wait for it (it cannot tell the
  // addresses apart).  All loads are waited for before each barrier.
  // Physical page of this wave's rows of tile `tile` (paged form).
  auto page_of = [&](int tile) -> int {
    if constexpr (kPaged) {
      tile = min(tile, ntiles - 1);
      // Staged entries: 0 .. min(last page of the tiles, max_pages, limit).
      const int lp = min((tile * kBN + 8 * wv) >> p.page_shift,
                         min(p.max_pages, kPrefillMaxPages) - 1);
      return __builtin_amdgcn_readfirstlane(sPage[lp]);
    } else {
      return 0;
    }
  };
  auto tile_load_part = [&](int kv, int buf, int tile, int i, int pg) {
    tile = min(tile, ntiles - 1);
    u32x4 rsrc;
    if constexpr (kPaged) {
      const int row0 = tile * kBN + 8 * wv;
      const int valid = min(max(S_kv - row0, 0), 8);
      const size_t e = ((size_t)pg * p.H_kv + kvh) * ((size_t)kD << p.page_shift) +
                       (size_t)(row0 & ((1 << p.page_shift) - 1)) * kD;
      const uintptr_t a = reinterpret_cast<uintptr_t>((kv ? Vg : Kg) + e) -
                          (uintptr_t)(8 * wv) * (kD * 2);
      rsrc = buffer_rsrc(reinterpret_cast<const void*>(a), (unsigned)(8 * wv + valid) * (kD * 2));
    } else {
      rsrc = buffer_rsrc((kv ? Vg : Kg) + (size_t)tile * (kBN * kD),
                         (unsigned)min(S_kv - tile * kBN, kBN) * (kD * 2));
    }
    dma_load_x4(ld_off[kv][i], rsrc,
                (kv ? lds_v0 : lds_k0) + buf * kTileBytes + 4 * (kInsts * wave + i) * kD * 2);
  };
  auto tile_load = [&](int kv, int buf, int tile) {
    const int pg = page_of(tile);
#pragma unroll
    for (int i = 0; i < kInsts; ++i) tile_load_part(kv, buf, tile, i, pg);
  };

  // S^T of one tile from K buffer `kb`.
  auto compute_s = [&](Tile16& T, int kb) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const f32x16 zero = {};
        T.s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_opnd(kb, mt, ks), qb[ks],
                                                          ks ? T.s[mt] : zero, 0, 0, 0);
      }
  };

  // S^T of tile `tile` with the K operands read from global memory (the
  // rare fix-up path): the same operand values and MFMA sequence as
  // compute_s, so the scores are bit-identical, but no LDS slot is read --
  // the waves are not synchronised between the two steps of a group, and
  // another wave may already be refilling the slot that held this tile.
  // Rows past S_kv read row S_kv - 1 (in bounds); their scores are masked.
  auto compute_s_global = [&](Tile16& T, int tile) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int row = min(tile * kBN + 32 * mt + c, S_kv - 1);
      const __bf16* kr;
      if constexpr (kPaged) {
        const int lp = min(row >> p.page_shift, min(p.max_pages, kPrefillMaxPages) - 1);
        kr = Kg + ((size_t)sPage[lp] * p.H_kv + kvh) * ((size_t)kD << p.page_shift) +
             (size_t)(row & ((1 << p.page_shift) - 1)) * kD;
      } else {
        kr = Kg + (size_t)row * kD;
      }
      kr += 8 * h2;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const f32x16 zero = {};
        T.s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(kr + 16 * ks)), qb[ks],
                                                          ks ? T.s[mt] : zero, 0, 0, 0);
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
  auto pv = [&](const PTile& P, int vb) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_opnd(vb, st, dt), P.p[st], o[dt], 0, 0,
                                                        0);
  };

  float m_ref = kNegInf;  // reference max (log2 domain) of row qrow, same on both halves
  float lpart = 0.f;      // this lane's half of the running sum
  // |scale| * log2(e), kept away from zero so that masked (-inf) scores
  // still give -inf; for |scale * q.k| far below 2^-24 * 32 the weights are
  // the same as with the exact scale.
  const float sl2 = fmaxf(p.scale_log2, 1e-30f);
  const int vis_last = p.causal ? offset + qrow : S_kv - 1;

  auto mask_tile = [&](Tile16& T, int tile) {
    const int kbase = tile * kBN;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kbase + 32 * mt + 8 * (i >> 2) + 4 * h2 + (i & 3);
        if (key > vis_last || key >= S_kv) T.s[mt][i] = kNegInf;
      }
  };

  auto half_max = [&](const f32x16& s) {
    float r = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) r = fmaxf(r, s[i]);
    return r;
  };

  // Moves the reference to 32 below the row max when that max (log2 units,
  // `hscaled` per lane) exceeds the reference by more than 64, rescaling O
  // and l, which are kept relative to the reference.
  auto move_ref = [&](float hscaled) {
    const float rmax = wave_max_xor(hscaled, 32);
    const float m_new = rmax > m_ref + kResetGap ? rmax - kRefBelow : m_ref;
    const float corr = fast_exp2(m_ref - m_new);
    lpart *= corr;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= corr;
    m_ref = m_new;
  };

  // P = exp2(S*scale - ref) rounded to bf16; returns the fp32 sum of P over
  // this lane's 32 keys (masked scores are -inf and give 0).
  auto exps = [&](const Tile16& T, PTile& P) -> float {
    const float negr = -m_ref;
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      u32x4 pw;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float e0 = fast_exp2(__builtin_fmaf(T.s[st >> 1][8 * (st & 1) + 2 * jj], sl2, negr));
        const float e1 =
            fast_exp2(__builtin_fmaf(T.s[st >> 1][8 * (st & 1) + 2 * jj + 1], sl2, negr));
        psum += e0 + e1;
        pw[jj] = pack_bf16x2(e0, e1);
      }
      P.p[st] = as_bf16x8(pw);
    }
    return psum;
  };

  // One step's matrix work: the 32 MFMAs of P.V(j-1) and S(j+1) in one
  // sequence, each MFMA's LDS operand read three MFMAs ahead, with the
  // softmax of tile j (P = exp2(S*scale - ref), rounded to bf16; fp32 row
  // sums) spread between them so that the matrix unit and the vector ALUs
  // work at the same time.  Order: the 16 MFMAs of P.V(j-1), then S(j+1)
  // rows 0-31 (reusing the registers of S(j) rows 0-31), then rows 32-63
  // (in the registers of P(j-1), free once the P.V MFMAs have read it).
  // Exponential k of S(j) runs in slot k, one per MFMA: rows 0-31 finish
  // by slot 15, before their registers are overwritten, and rows 32-63
  // stay live to the end of the sequence.  Two waves share a SIMD and run
  // the same sequence in step, so an even spread keeps the vector port's
  // load per slot below one MFMA's duration.  Returns this lane's fp32 sum
  // of P(j).
  // `ld` (when not null) lists two tile loads as {kv, buffer, tile, page}
  // entries; their four instructions are spread over the sequence (one
  // every eighth MFMA) so that the load path is fed gradually instead of
  // stalling the waves at the start of the group.
  auto mma_step = [&](auto kbuf, auto vbuf, Tile16& T, const PTile& Pprev, PTile& Pcur,
                      const int (*ld)[4]) {
    constexpr int kb = decltype(kbuf)::value;
    constexpr int vb = decltype(vbuf)::value;
    auto opnd = [&](int i) -> bf16x8 {
      if (i < 16) return v_opnd(vb, i >> 2, i & 3);
      if (i < 24) return k_opnd(kb, 0, i - 16);
      return k_opnd(kb, 1, i - 24);
    };
    float negr = -m_ref;
    // Anchor the softmax inputs here, so that no exponential is hoisted
    // out of the sequence.
    asm volatile("" : "+v"(negr));
    float psum = -0.f;   // -0 + x == x for every x, so the first add folds away
    u32x4 pw[4];
    float ev[32];   // exponentials of S(j), key order of the lane's scores
    Tile16 Sn;
    constexpr int kAhead = 3;   // operand reads in flight ahead of the MFMA
    bf16x8 ring[kAhead + 1];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) ring[i] = opnd(i);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      // One slot per MFMA: the scheduler may not move work between slots.
      __builtin_amdgcn_sched_barrier(0);
      if (i + kAhead < 32) ring[(i + kAhead) % (kAhead + 1)] = opnd(i + kAhead);
      if (ld != nullptr && (i & 7) == 2) {
        const int* l = ld[i >> 4];
        tile_load_part(l[0], l[1], l[2], (i >> 3) & 1, l[3]);
      }
      const bf16x8 a = ring[i % (kAhead + 1)];
      const f32x16 zero = {};
      if (i < 16) {
        o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, Pprev.p[i >> 2], o[i & 3], 0, 0, 0);
      } else if (i < 24) {
        Sn.s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[i - 16], i > 16 ? Sn.s[0] : zero,
                                                          0, 0, 0);
      } else {
        Sn.s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[i - 24], i > 24 ? Sn.s[1] : zero,
                                                          0, 0, 0);
      }
      // Exponential k (score k of the lane: rows 32*(k/16).., key 32*(k/16)
      // + 8*((k%16)/4... as S.s[k/16][k%16]) runs in slot k.
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        if (k != i) continue;
        ev[k] = fast_exp2(__builtin_fmaf(T.s[k >> 4][k & 15], sl2, negr));
        if ((k & 1) == 0) {
          // Keep this exponential in this slot (not sunk towards its use).
          asm volatile("" ::"v"(ev[k]));
          continue;
        }
        // Pair k/2 complete: keys 32*mt + 8*(q/4) + 4*h2 + 2*(q%4) + {0, 1}
        // of S(j) rows 32*mt.., q = (k/2) % 8.
        const int mt = k >> 4, q = (k >> 1) & 7;
        psum += ev[k - 1] + ev[k];
        const unsigned w = pack_bf16x2(ev[k - 1], ev[k]);
        asm volatile("" ::"v"(w), "v"(psum));
        pw[2 * mt + (q >> 2)][q & 3] = w;
        if ((q & 3) == 3) Pcur.p[2 * mt + (q >> 2)] = as_bf16x8(pw[2 * mt + (q >> 2)]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    T = Sn;
    return psum;
  };

  // Prologue: K tiles 0-2 and V tile 0 in LDS, V buffer 3 (read as tile
  // -1 by the first step, with P = 0) zeroed; S of tile 0.  The paged
  // form first stages the block-table entries of the pages its tiles touch.
  if constexpr (kPaged) {
    const int n_lp = min(min(((ntiles * kBN - 1) >> p.page_shift) + 1, p.max_pages),
                         kPrefillMaxPages);
    const int* trow = p.block_table + (size_t)b * p.max_pages;
    for (int i = t; i < n_lp; i += kThreads) sPage[i] = min(max(trow[i], 0), p.num_pages - 1);
    __syncthreads();
  }
  tile_load(0, 0, 0);
  if (ntiles > 1) tile_load(0, 1, 1);
  if (ntiles > 2) tile_load(0, 2, 2);
  tile_load(1, 0, 0);
  {
    u32x4* z = reinterpret_cast<u32x4*>(sV[3]);
    for (int i = t; i < kTileElems / 8; i += kThreads) z[i] = u32x4{0, 0, 0, 0};
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // this wave's tile loads landed
  __syncthreads();
  Tile16 T;
  PTile PA, PB;
#pragma unroll
  for (int st = 0; st < 4; ++st) PB.p[st] = as_bf16x8(u32x4{0, 0, 0, 0});
  compute_s(T, 0);
  __syncthreads();                      // every wave has read K tile 0
  // The reference starts 32 below the row max of tile 0's visible scores
  // (every row sees key 0), so the first step does not take the fix-up
  // path.  The mask is idempotent: step 0 applies it again.
  if (n_full == 0) mask_tile(T, 0);
  move_ref(fmaxf(half_max(T.s[0]), half_max(T.s[1])) * sl2);

  // Step j: P.V of tile j-1, the softmax of tile j (scores in T) into
  // `pcur`, and S of tile j+1 into T.  Tiles past the wave's last visible
  // one are fully masked (P = 0), so every step runs the same sequence.
  // The softmax uses the current reference; if any weight exceeds 2^64
  // (some score is more than 64 above the reference: rare once the
  // prologue has set it from tile 0) the lane sum shows it, and the tile's
  // scores are recomputed from K in global memory, the reference moved and
  // P redone.
  auto step = [&](auto kbuf, auto vbuf, PTile& pprev, PTile& pcur, int j, const int (*ld)[4]) {
    if (j >= n_full) mask_tile(T, j);
    float psum = mma_step(kbuf, vbuf, T, pprev, pcur, ld);
    if (__any(!(psum <= kPsumLimit))) {
      Tile16 Tj;
      compute_s_global(Tj, j);
      if (j >= n_full) mask_tile(Tj, j);
      const float hmax = fmaxf(half_max(Tj.s[0]), half_max(Tj.s[1]));
      move_ref(hmax * sl2);
      psum = exps(Tj, pcur);
    }
    lpart += psum;
  };
  // Group of steps j, j+1 (j % 4 == 2*G): reads K tiles j+1, j+2 and V
  // tiles j-1, j; loads V tiles j+1, j+2 during step j and K tiles j+3,
  // j+4 during step j+1 (K tile j stays in LDS through step j, K tile j+1
  // through step j+1), all into buffers the previous group read; one
  // barrier at the end.
  auto group = [&](auto gsel, int j) {
    constexpr int G = decltype(gsel)::value;
    const int ldv[2][4] = {{1, (2 * G + 1) % 4, j + 1, page_of(j + 1)},
                           {1, (2 * G + 2) % 4, j + 2, page_of(j + 2)}};
    const int ldk[2][4] = {{0, (2 * G + 3) % 4, j + 3, page_of(j + 3)},
                           {0, (2 * G + 4) % 4, j + 4, page_of(j + 4)}};
    step(Int<(2 * G + 1) % 4>(), Int<(2 * G + 3) % 4>(), PB, PA, j, ldv);
    if (j + 1 < ntiles) {
      step(Int<(2 * G + 2) % 4>(), Int<(2 * G) % 4>(), PA, PB, j + 1, ldk);
    } else {
      tile_load(0, (2 * G + 3) % 4, j + 3);
      tile_load(0, (2 * G + 4) % 4, j + 4);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
  };
  for (int j = 0; j < ntiles; j += 4) {
    group(Int<0>(), j);
    if (j + 2 < ntiles) group(Int<1>(), j + 2);
  }
  // P.V of the last tile: its P is in PA (even tile) or PB (odd tile).
  {
    const int last = ntiles - 1;
    pv((last & 1) ? PB : PA, last & 3);
  }

  // Epilogue: O = O / l, rounded to bf16.  Lane holds, for d-tile dt and
  // i = 0..15, d = 32*dt + 8*(i/4) + 4*h2 + (i%4) of row qw0 + c: 8-byte
  // pieces of 32 rows.  Stored as they are, every store instruction would
  // touch 32 rows; instead each wave stages its 32 rows (8 KiB, 16-byte
  // pieces XOR-swizzled by row) in the K ring, which nothing reads any more
  // (the last group's barrier followed its last use), and copies them out
  // row-contiguous: 4 whole rows per store instruction.
  // The ids and the kernel arguments are re-read through opaque copies (the
  // arguments from the kernarg segment, where this kernel's only argument
  // sits at offset 0), so the row addressing is recomputed here rather than
  // held in registers through the loop.
  int tid_e = threadIdx.x, bid_e = vid;
  typedef const __attribute__((address_space(4))) PrefillParams KernargParams;
  KernargParams* pk = (KernargParams*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+v"(tid_e), "+s"(bid_e), "+s"(pk));
  const auto& pa = *pk;   // fields read with scalar loads where used below
  const int lane_e = tid_e & 63, c_e = tid_e & 31, h2_e = (tid_e >> 5) & 1;
  const int wave_e = __builtin_amdgcn_readfirstlane(tid_e >> 6);
  const Place pe = locate(pa, bid_e, wave_e);
  const float lsum = lpart + __shfl_xor(lpart, 32, 64);
  const float inv = 1.f / lsum;
  char* stage = reinterpret_cast<char*>(&sK[0][0]) + wave_e * (32 * kD * 2);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int pc = 4 * dt + i4;   // 16-byte piece of d = 32*dt + 8*i4 .. +8
      u32x2 v2 = {pack_bf16x2(o[dt][4 * i4] * inv, o[dt][4 * i4 + 1] * inv),
                  pack_bf16x2(o[dt][4 * i4 + 2] * inv, o[dt][4 * i4 + 3] * inv)};
      *reinterpret_cast<u32x2*>(stage + c_e * (kD * 2) + 16 * (pc ^ (c_e & 15)) + 8 * h2_e) = v2;
    }
  {
    const int pc = lane_e & 15;
    __bf16* obase = static_cast<__bf16*>(pa.o);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 4 * k + (lane_e >> 4);
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * (kD * 2) + 16 * (pc ^ (r & 15)));
      if (pe.qw0 + r < pe.S_q)
        *reinterpret_cast<u32x4*>(obase + (pe.qrow0 + (size_t)(pe.qw0 + r) * pe.qstride) * kD +
                                  8 * pc) = v;
    }
  }
  const int qrow_e = pe.qw0 + c_e;
  if (qrow_e < pe.S_q && pa.lse != nullptr && h2_e == 0)
    pa.lse[pe.qrow0 + (size_t)qrow_e * pe.qstride] = (m_ref + __log2f(lsum)) * kLn2;
  };

  // Causal dense launches pair each query block with its mirror (the
  // heaviest with the lightest, ...), so every workgroup does about the
  // same work and the grid has half as many workgroups.  A block's id is
  // its workgroup id in the unpaired grid; the second one is derived from an
  // opaque copy of the workgroup id, so nothing of the first block's
  // addressing stays live through it.
  if (kVarlen || !p.pair_blocks) {
    run_block((int)blockIdx.x);
    return;
  }
  {
    const int per_rank = p.H_kv * (p.G / p.heads_per_wg) * p.B;
    run_block((int)(blockIdx.x % per_rank + per_rank * (blockIdx.x / per_rank)));
  }
  int bid2 = blockIdx.x;
  asm volatile("" : "+s"(bid2));
  typedef const __attribute__((address_space(4))) PrefillParams KernargParams2;
  KernargParams2* pk2 = (KernargParams2*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(pk2));
  const int per_rank2 = pk2->H_kv * (pk2->G / pk2->heads_per_wg) * pk2->B;
  const int rank2 = pk2->n_qblk - 1 - bid2 / per_rank2;
  if (rank2 == bid2 / per_rank2) return;   // the middle block of an odd count
  __syncthreads();   // the first block's output staging in sK has been read
  run_block(bid2 % per_rank2 + per_rank2 * rank2);
}

// Tile count of a varlen work item (b, pblk): the key tiles its workgroup
// walks (0 past the chunk's end).  Mirrors the extent computed in the
// attention kernel.
// `cu` and `lens` are the length arrays, in LDS or in global memory.
__device__ __forceinline__ int varlen_item_cost(const PrefillParams& p, const int* cu,
                                                const int* lens, int item) {
  const int b = item / p.n_qblk, pblk = item % p.n_qblk;
  const int t0 = min(max(cu[b], 0), p.S_q);
  const int t1 = min(max(cu[b + 1], t0), p.S_q);
  const int S_q = t1 - t0;
  const int S_kv = min(max(lens[b], 0), p.S_kv);
  const int rows = 32 * (kWaves / p.heads_per_wg);
  const int P0 = pblk * rows;
  if (P0 >= S_q) return 0;
  int kend = S_kv;
  if (p.causal) kend = min(kend, max(S_kv - S_q, 0) + P0 + rows);
  return (kend + kBN - 1) / kBN;
}

constexpr int kSchedThreads = 256;
constexpr int kSchedBins = 2048;
constexpr int kSchedPer = kSchedBins / kSchedThreads;   // bins per thread in the scan
constexpr int kSchedStagedB = 4096;   // batches up to this size read their lengths from LDS

// The varlen work list: every item b * n_qblk + pblk, ordered by tile count
// (bins of 2^shift tiles), heaviest first.  One workgroup of 4 waves: the
// lengths staged in LDS (batches of up to kSchedStagedB sequences; larger
// ones read them from global memory), a histogram of the bins in LDS, a
// descending exclusive scan (each thread sums 8 bins, a shuffle scan within
// each wave, then the wave totals), and each item placed at its bin's
// cursor.  Items within a bin land in any order; the result of each item
// does not depend on when it runs.
template <bool kStaged>
__device__ __forceinline__ void varlen_schedule(const PrefillParams& p, int* list, int shift,
                                                int* hist, int* wsum, const int* cu,
                                                const int* lens) {
  const int t = threadIdx.x;
  const int n = p.B * p.n_qblk;
  auto bin_of = [&](int item) {
    return min(varlen_item_cost(p, cu, lens, item) >> shift, kSchedBins - 1);
  };
  const int lane = t & 63, wave = t >> 6;
  // Most items of a ragged batch lie past their chunk's end (bin 0): that
  // bin is counted and filled one wave at a time (a ballot and one atomic),
  // so its items do not serialise on one LDS address.
  for (int i0 = 0; i0 < n; i0 += kSchedThreads) {
    const int i = i0 + t;
    const int bin = i < n ? bin_of(i) : -1;
    const unsigned long long zero = __ballot(bin == 0);
    if (bin > 0) atomicAdd(&hist[bin], 1);
    if (lane == 0 && zero != 0) atomicAdd(&hist[0], __popcll(zero));
  }
  __syncthreads();
  // Descending order: thread t owns bins NB-1-8t .. NB-8-8t.
  int local[kSchedPer], sum = 0;
#pragma unroll
  for (int j = 0; j < kSchedPer; ++j) {
    local[j] = hist[kSchedBins - 1 - (kSchedPer * t + j)];
    sum += local[j];
  }
  int incl = sum;   // inclusive scan of the thread sums within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = incl - sum;
  for (int w = 0; w < wave; ++w) base += wsum[w];
#pragma unroll
  for (int j = 0; j < kSchedPer; ++j) {
    hist[kSchedBins - 1 - (kSchedPer * t + j)] = base;   // becomes the bin's cursor
    base += local[j];
  }
  __syncthreads();
  // Both passes bin each item alike (the length arrays are read-only
  // meanwhile), so every position is below n; the bound only guards the list.
  for (int i0 = 0; i0 < n; i0 += kSchedThreads) {
    const int i = i0 + t;
    const int bin = i < n ? bin_of(i) : -1;
    const unsigned long long zero = __ballot(bin == 0);
    int zbase = 0;
    if (lane == 0 && zero != 0) zbase = atomicAdd(&hist[0], __popcll(zero));
    zbase = __shfl(zbase, 0, 64);
    int pos = n;
    if (bin == 0) {
      pos = zbase + __popcll(zero & ((1ull << lane) - 1ull));
    } else if (bin > 0) {
      pos = atomicAdd(&hist[bin], 1);
    }
    if (pos < n) list[pos] = i;
  }
}

__global__ __launch_bounds__(kSchedThreads) void prefill_varlen_schedule_kernel(PrefillParams p,
                                                                               int* list,
                                                                               int shift) {
  __shared__ int hist[kSchedBins];
  __shared__ int wsum[kSchedThreads / 64];
  __shared__ int s_cu[kSchedStagedB + 1], s_len[kSchedStagedB];
  const int t = threadIdx.x;
  for (int i = t; i < kSchedBins; i += kSchedThreads) hist[i] = 0;
  if (p.B <= kSchedStagedB) {
    for (int i = t; i <= p.B; i += kSchedThreads) s_cu[i] = p.cu_seqlens_q[i];
    for (int i = t; i < p.B; i += kSchedThreads) s_len[i] = p.kv_lens[i];
    __syncthreads();
    varlen_schedule<true>(p, list, shift, hist, wsum, s_cu, s_len);
  } else {
    __syncthreads();
    varlen_schedule<false>(p, list, shift, hist, wsum, p.cu_seqlens_q, p.kv_lens);
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
  const long long nblk = p.pair_blocks && p.cu_seqlens_q == nullptr ? (p.n_qblk + 1) / 2 : p.n_qblk;
  const long long nwg = nblk * p.B * p.H_kv * (p.G / p.heads_per_wg);
  if (p.cu_seqlens_q != nullptr) {
    int shift = 0;
    while ((((long long)p.S_kv + kBN - 1) / kBN >> shift) >= kSchedBins) ++shift;
    hipLaunchKernelGGL(prefill_varlen_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, p,
                       p.sched, shift);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.block_table != nullptr) {
      hipLaunchKernelGGL((prefill_bf16_kernel<true, true>), dim3((unsigned)nwg), dim3(kThreads), 0,
                         stream, p);
    } else {
      hipLaunchKernelGGL((prefill_bf16_kernel<true, false>), dim3((unsigned)nwg), dim3(kThreads),
                         0, stream, p);
    }
  } else {
    hipLaunchKernelGGL((prefill_bf16_kernel<false, false>), dim3((unsigned)nwg), dim3(kThreads), 0,
                       stream, p);
  }
  return hipGetLastError();
}

}  // namespace gqa
