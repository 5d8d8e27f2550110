// Decode attention (T_q = 1) for gfx950: split-KV partial kernels and the
// log-sum-exp combine.
//
// Method: ADR-0060 "AHBM GQA Fused Attention Kernel (Llama3-70B)", revision
// 5a76ed4 -- §5.2 (the G query heads of one KV head are folded into the GEMM
// M dimension so each K/V tile is streamed once for all of them), §3 (the
// per-tile online-softmax update), §4 (splits produce unnormalised
// (m, l, O) partials merged by the associative log-sum-exp merge, with one
// normalisation at the end) and §2.1 (contiguous position blocks per split).
//
// GPU mapping.  One workgroup = 4 waves = one contiguous split of
// `chunk` keys of one (sequence, KV head); wave w sweeps the w-th quarter of
// the split in blocks of 32 keys, straight from HBM into registers (K and V
// are read exactly once, so they bypass LDS).  Each wave reads one address
// stream: the K rows of two blocks, then their V rows, and so on, with the
// online-softmax update once per two blocks.  Scores are computed
// transposed, S^T = K . Q^T, on the 16x16x32 bf16 MFMA with keys in M and
// the (zero-padded) G <= 16 query heads in N; O^T = V^T . P^T uses the same
// MFMA with d in M.  The 8x8 transpose V needs is done in registers by byte
// permutes.  Scores live in the log2 domain (scale * log2(e) folded into one
// multiply) so the exponentials are single v_exp_f32 instructions.  The 4
// waves merge through LDS and the workgroup writes one partial.
//
// A second kernel merges the partials: one wave per (sequence, query head)
// and quarter of d, so a row's partials come in through four CUs' load
// pipelines at once.  The one-launch form (decode_fused_bf16_kernel and the
// fp32 split kernel with DecodeParams::counters set) merges inside the
// split kernel instead -- the last workgroup to arrive for a (sequence, KV
// head) merges the others' partials -- and is slower on MI355X: publishing
// partials across the 8 XCDs' separate L2s costs agent-coherent stores and
// an atomic per workgroup, and the merge then runs on one CU per head.

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace gqa {

namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kBlk = 32;  // keys per wave step

// One lane's loads of one 32-key block of K or of V: eight 16-byte pieces
// (a register slot holds either).
//   K: piece 4*sb + kb = K row (key0 + 16*sb + l%16), d range
//      32*kb + 8*(l/16) .. +8 -> A operand of S^T tile sb, k-step kb.
//   V: piece j = V row key(g, j), d range 8*(l%16) .. +8, where
//      key(g, j) = 4g + j (j < 4) or 16 + 4g + (j - 4) (j >= 4): the keys
//      this lane's P^T slots hold.
typedef u32x4 Slot[8];

// Per-lane byte offsets of a block's loads relative to the block's first
// key (the block's own offset is added to them).
struct BlockOffsets {
  int k[2];   // K row l%16 (+16 rows for sb = 1), d = 8*(l/16)
  int v[2];   // V row 4*(l/16) (+16 rows for j >= 4), d = 8*(l%16)
};

// Running state of one wave: query n = lane % 16 (rows >= G are padding).
struct State {
  float m;       // running max of log2-domain scores (same on the 4 lanes of n)
  float l;       // this lane's share of the running sum of p
  f32x4 o[8];    // O^T, d-tile dt: lane holds d = 8*(4*(lane/16)+i) + dt, query n
};

// S^T = K . Q^T for the block's two 16-key sub-blocks.
__device__ __forceinline__ void block_scores(f32x4 (&s)[2], const Slot& k, const bf16x8 (&qb)[4]) {
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    s[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      s[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[4 * sb + kb]), qb[kb], s[sb], 0, 0, 0);
  }
}

// O^T += V^T . P^T.  V^T operand for d-tile dt: element j =
// V[key(g, j)][8*(lane%16) + dt].
__device__ __forceinline__ void block_pv(State& st, const Slot& v, bf16x8 pb) {
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const int w = dt >> 1;
    u32x4 a;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const unsigned int lo = v[2 * jj][w];
      const unsigned int hi = v[2 * jj + 1][w];
      // One byte permute: the low (dt even) or high (dt odd) halves of
      // lo and hi, lo's in the low half of the result.
      a[jj] = __builtin_amdgcn_perm(hi, lo, (dt & 1) ? 0x07060302u : 0x05040100u);
    }
    st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), pb, st.o[dt], 0, 0, 0);
  }
}

// Online log-sum-exp merge of split partials, NG at a time per lane so that
// all of a group's loads are in flight together.  (M, acc, lacc) is the running
// state; a group is folded in with the merge rule of §4: rescale both sides
// to the larger max and add.
struct MergeAcc {
  float M;
  f32x4 acc;
  float lacc;
};

constexpr int kCombSlots = 8;     // split slots per wave (lane / 8)

template <int NG>   // splits per lane and load round
struct MergeLoads {
  float m[NG], l[NG];
  f32x4 o[NG];
};

// Loads splits s0, s0 + stride, ...; indices at or past `s_alloc` (the
// partials the workspace holds per row) re-read the last one, so every load
// is unconditional and all of them are in flight together.  Such splits lie
// past the sequence's split count and are discarded by merge_fold.
template <int NG>
__device__ __forceinline__ void merge_load(MergeLoads<NG>& g, const float* ml, const float* po, int s0,
                                           int s_alloc, int stride) {
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    const int s = min(s0 + u * stride, s_alloc - 1);
    const f32x2 m2 = *reinterpret_cast<const f32x2*>(ml + 2 * s);
    g.o[u] = *reinterpret_cast<const f32x4*>(po + (size_t)s * kD);
    g.m[u] = m2[0];
    g.l[u] = m2[1];
  }
}

// Merges (m, acc, l) into `st` with the rule of §4.  Branch-free: with both
// sides empty (m = -inf) the reference is 0 and both weights are 0.
__device__ __forceinline__ void merge_pair(MergeAcc& st, float m, f32x4 acc, float l) {
  const float gm = fmaxf(st.M, m);
  const float ref = gm == kNegInf ? 0.f : gm;
  const float c0 = fast_exp2(st.M - ref);
  const float c1 = fast_exp2(m - ref);
  st.acc = st.acc * c0 + acc * c1;
  st.lacc = st.lacc * c0 + l * c1;
  st.M = gm;
}

// Folds the loaded splits below `s_valid` (the splits of this call) into
// `st`; the others are replaced by the identity (-inf, 0, 0) before use.
template <int NG>
__device__ __forceinline__ void merge_fold(MergeAcc& st, MergeLoads<NG>& g, int s0, int s_valid,
                                           int stride) {
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    if (s0 + u * stride >= s_valid) {
      g.m[u] = kNegInf;
      g.l[u] = 0.f;
      g.o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  float gm = st.M;
#pragma unroll
  for (int u = 0; u < NG; ++u) gm = fmaxf(gm, g.m[u]);
  // Branch-free (so that no load is sunk behind a branch): with every side
  // empty, gm = -inf and the weights below are exp2(-inf) = 0.
  const float ref = gm == kNegInf ? 0.f : gm;
  const float c = fast_exp2(st.M - ref);
  st.acc *= c;
  st.lacc *= c;
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    const float w = fast_exp2(g.m[u] - ref);
    st.acc += w * g.o[u];
    st.lacc += w * g.l[u];
  }
  st.M = gm;
}

// What a merge's first load round needs.  The combine launch passes these
// as kernel arguments of their own, ahead of DecodeParams, and this file is
// built with kernel-argument preloading, so they arrive in registers with
// the wave: the first loads issue without waiting for the argument block.
struct CombineHead {
  const int32_t* kv_lens;
  const float* ws_o;
  const float* ws_ml;
  int n_split_max;
  int rows_per_seq;   // H_q * T_q
};

// Combine: one wave per (output row, quarter of d), rows being (sequence,
// query head, token); the 4 waves of a row run on different CUs, so a row's
// partials are fetched by four load pipelines at once.  Lane l takes split
// slot j = l / 8 (splits j, j + 8, j + 16, ...) and output columns
// 32*quarter + 4*(l % 8) .. +4; the 8 slots then merge across lanes
// (xor 8, 16, 32).  Normalises once and rounds to the output dtype (the
// final O / l of §4).  The first 8*NG splits' loads are issued together with
// the sequence length's, so a call of up to 8*NG splits costs one memory
// round trip; splits past the sequence's count are discarded after the
// loads.  NG (2, 4 or 8) follows the workspace's split count, so that a row
// with few splits does not load the same partial several times.
template <typename OutT, int NG, int U>
__device__ __forceinline__ void combine_rows(const DecodeParams& p, const CombineHead& hd, const int (&bh)[U],
                                             const int (&quarter)[U], int count, int lane) {
  // U (row, quarter) units, count of them valid: the first load round of
  // every unit is issued before any is folded, so the units share one
  // memory round trip; each unit's arithmetic is the same sequence as
  // with U = 1.
  const int slot = lane >> 3;
  MergeLoads<NG> g[U];
  int len[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u < count) {
      const size_t part0 = (size_t)bh[u] * hd.n_split_max;
      len[u] = hd.kv_lens[bh[u] / hd.rows_per_seq];
      merge_load(g[u], hd.ws_ml + 2 * part0, hd.ws_o + part0 * kD + 32 * quarter[u] + 4 * (lane & 7),
                 slot, hd.n_split_max, kCombSlots);
    }
  }
  // The first round's loads are issued before anything reads the other
  // parameters (whose loads would otherwise go first and be waited for).
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u >= count) break;
    const int d0 = 32 * quarter[u] + 4 * (lane & 7);
    const size_t part0 = (size_t)bh[u] * p.n_split_max;
    const float* ml = p.ws_ml + 2 * part0;
    const float* po = p.ws_o + part0 * kD + d0;
    const int L = min(len[u], p.max_kv_len);
    const int ns = (L + p.chunk - 1) / p.chunk;
    MergeAcc st{kNegInf, {0.f, 0.f, 0.f, 0.f}, 0.f};
    merge_fold(st, g[u], slot, ns, kCombSlots);
    for (int s0 = slot + kCombSlots * NG; s0 < ns; s0 += kCombSlots * NG) {
      merge_load(g[u], ml, po, s0, p.n_split_max, kCombSlots);
      merge_fold(st, g[u], s0, ns, kCombSlots);
    }
#pragma unroll
    for (int mask = 8; mask < 64; mask <<= 1) {
      f32x4 ao;
#pragma unroll
      for (int i = 0; i < 4; ++i) ao[i] = __shfl_xor(st.acc[i], mask, 64);
      const float mo = __shfl_xor(st.M, mask, 64);
      const float lo = __shfl_xor(st.lacc, mask, 64);
      merge_pair(st, mo, ao, lo);
    }
    if (slot == 0) {
      const float inv = 1.f / st.lacc;
      OutT* o = static_cast<OutT*>(p.o) + (size_t)bh[u] * kD + d0;
      if constexpr (sizeof(OutT) == 2) {
        const u32x2 w = {pack_bf16x2(st.acc[0] * inv, st.acc[1] * inv),
                         pack_bf16x2(st.acc[2] * inv, st.acc[3] * inv)};
        *reinterpret_cast<u32x2*>(o) = w;
      } else {
        *reinterpret_cast<f32x4*>(o) = st.acc * inv;
      }
      if (p.lse != nullptr && lane == 0 && quarter[u] == 0)
        p.lse[bh[u]] = (st.M + __log2f(st.lacc)) * kLn2;
    }
  }
}

template <typename OutT, int NG>
__device__ __forceinline__ void combine_row(const DecodeParams& p, const CombineHead& hd, int bh, int quarter,
                                            int lane) {
  const int bhs[1] = {bh}, qs[1] = {quarter};
  combine_rows<OutT, NG, 1>(p, hd, bhs, qs, 1, lane);
}

// Splits per lane and load round of the merge for a workspace of
// `n_split_max` partials per row (the combine launch uses the same rule).
__host__ __device__ constexpr int combine_ng(int n_split_max) {
  return n_split_max <= 16 ? 2 : n_split_max <= 32 ? 4 : 8;
}

// A partial value: a plain store for the combine launch; for the fused
// merge an agent-scope store, which writes through this XCD's L2 so that a
// workgroup on another XCD can read it.
__device__ __forceinline__ void store_partial(float* dst, float v, bool fused) {
  if (fused) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *dst = v;
}

// Fused merge, run by every thread of a split workgroup after its partial
// stores (the data-driven reduction of §4.3: no launch boundary between the
// sweeps and the merge).  The partials were stored with agent-scope
// (write-through) stores, and each thread waits until its own are
// acknowledged -- that is what makes them visible on the other XCDs, whose
// L2 caches are separate, without writing back a whole L2 as a release
// fence would.  The workgroup then counts itself in, and the workgroup that
// arrives last -- the one that sees n_split - 1 earlier arrivals --
// invalidates its caches (an agent-scope acquire), merges the partials with
// exactly the combine launch's code (so the results are bit-identical to
// it), and resets the counter to zero for the next call.  `n_split` is this
// sequence's split count: workgroups past its end return before writing a
// partial and are not counted.
template <typename OutT>
__device__ __forceinline__ void fused_merge_tail(const DecodeParams& p, int b, int kvh,
                                                 int n_split) {
  __shared__ int s_last;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(p.counters + (size_t)b * p.H_kv + kvh, 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(n_split - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int M = p.G * p.T_q;
  const int row0 = (b * p.H_q + kvh * p.G) * p.T_q;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int nwaves = blockDim.x >> 6;
  // Wave w takes units w, w + nwaves, ... in batches whose first load
  // rounds are all in flight together (at most ~96 registers of loads).
  const int ng = combine_ng(p.n_split_max);
  const CombineHead hd{p.kv_lens, p.ws_o, p.ws_ml, p.n_split_max, p.H_q * p.T_q};
  auto run = [&](auto ngc, auto uc) {
    constexpr int NG = decltype(ngc)::value, U = decltype(uc)::value;
    for (int base = wave; base < 4 * M; base += nwaves * U) {
      int bhs[U], qs[U], count = 0;
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int u = min(base + nwaves * i, 4 * M - 1);
        bhs[i] = row0 + (u >> 2);
        qs[i] = u & 3;
        count += base + nwaves * i < 4 * M;
      }
      combine_rows<OutT, NG, U>(p, hd, bhs, qs, count, lane);
    }
  };
  if (ng == 2) run(std::integral_constant<int, 2>(), std::integral_constant<int, 8>());
  else if (ng == 4) run(std::integral_constant<int, 4>(), std::integral_constant<int, 4>());
  else run(std::integral_constant<int, 8>(), std::integral_constant<int, 2>());
  if (threadIdx.x == 0)
    __hip_atomic_store(p.counters + (size_t)b * p.H_kv + kvh, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// The bf16 split sweep.  Grid: (n_split_max, H_kv, B); block: 256
// threads.  kPaged: K/V live in a page pool addressed through the block
// table (DecodeParams::block_table).  kFused: the one-launch decode
// (DecodeParams::counters set) merges the partials at the end.
template <bool kPaged, bool kFused>
__device__ __forceinline__ void decode_partial_bf16(const DecodeParams& p, int kv_len) {
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int lane = threadIdx.x & 63;
  const int quarter = p.chunk / kWaves;
  const int start = split * p.chunk;
  // Paged: lane j fetches the block-table entry of the wave's logical page
  // lp0 + j (at most 64 pages per wave range, checked on the host).  The
  // wave's first page follows from the split alone, so this load is issued
  // together with the sequence length's rather than after it; entries past
  // the table row are clamped to its last one, and those past the sequence
  // are not used.
  const int lp0 = (start + wave * quarter) >> p.page_shift;
  int pt_raw = 0;
  if constexpr (kPaged)
    pt_raw = p.block_table[(size_t)b * p.max_pages + min(lp0 + lane, p.max_pages - 1)];
  const int L = min(kv_len, p.max_kv_len);
  // Keeps the table load above the early exit below (the compiler would
  // otherwise sink it there, behind the length's round trip).
  if constexpr (kPaged) asm volatile("" : "+v"(pt_raw));
  if (start >= L) return;
  const int end = min(start + p.chunk, L);
  const int ws = start + wave * quarter;
  const int we = min(ws + quarter, end);

  const __bf16* q = static_cast<const __bf16*>(p.q);
  // Contiguous cache: this (sequence, KV head)'s rows (unused when paged).
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + (kPaged ? 0 : ((size_t)b * p.H_kv + kvh) * p.kv_cap * kD);
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + (kPaged ? 0 : ((size_t)b * p.H_kv + kvh) * p.kv_cap * kD);

  // Q^T operand: row n = lane%16 of this KV head's M = G*T_q folded rows
  // (row n is token n % T_q of head n / T_q; T_q = 1 for plain decode),
  // zero past M.  Row n sees keys up to L - T_q + n % T_q.
  const int n = lane & 15;
  const int g = lane >> 4;
  const int M = p.G * p.T_q;
  const size_t row0 = ((size_t)b * p.H_q + (size_t)kvh * p.G) * p.T_q;
  const bool row_ok = n < M;
  const int vis_last = row_ok ? L - p.T_q + n % p.T_q : L - 1;
  bf16x8 qb[4];
  {
    const __bf16* qrow = q + (row0 + (row_ok ? n : 0)) * kD + 8 * g;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qb[kb] = as_bf16x8(row_ok ? ld16(qrow + 32 * kb) : u32x4{0, 0, 0, 0});
  }

  State st;
  st.m = kNegInf;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (ws < we) {
    // Blocks of 32 keys; only the last one of the wave's range can be
    // partial (its keys past the range are masked).
    const int nblk = (we - ws + kBlk - 1) / kBlk;
    const unsigned bytes = kPaged ? 0u : (unsigned)(we - ws) * (kD * 2);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (size_t)ws * kD), (short)0, bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (size_t)ws * kD), (short)0, bytes, 0x00020000);
    BlockOffsets off;
    {
      const int r = lane & 15;
      off.k[0] = r * (kD * 2) + 16 * g;
      off.k[1] = off.k[0] + 16 * (kD * 2);
      off.v[0] = 4 * g * (kD * 2) + 16 * r;
      off.v[1] = off.v[0] + 16 * (kD * 2);
    }
    // Paged: lane j holds the physical page of the wave's logical page
    // lp0 + j, clamped into the pool.
    const int shift = p.page_shift;
    int pt = 0;
    if constexpr (kPaged) {
      const int npg = ((we - 1) >> shift) - lp0 + 1;
      if (lane < npg) pt = min(max(pt_raw, 0), p.num_pages - 1);
    }
    // Paged: the resources of block i's two 16-key sub-blocks.
    auto paged_rsrc = [&](const __bf16* base, int i, __amdgpu_buffer_rsrc_t (&r)[2])
                          __attribute__((always_inline)) {
      const size_t page_elems = (size_t)p.H_kv * (kD << shift);
      const size_t head_elems = (size_t)kvh * (kD << shift);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int pos = ws + i * kBlk + 16 * sb;
        // readfirstlane: the page is wave-uniform, and saying so keeps the
        // resources in scalar registers (no per-lane loop around the loads).
        const int pp = __builtin_amdgcn_readfirstlane(
            __builtin_amdgcn_readlane(pt, min((pos >> shift) - lp0, 63)));
        const size_t e = (size_t)pp * page_elems + head_elems + (size_t)(pos & ((1 << shift) - 1)) * kD;
        const unsigned nb = __builtin_amdgcn_readfirstlane((unsigned)max(0, min(16, we - pos)) * (kD * 2));
        r[sb] = __builtin_amdgcn_make_buffer_rsrc((void*)(base + e), (short)0, nb, 0x00020000);
      }
    };
    // One stream per wave.  The wave reads the K rows of a super-block of
    // kSblk blocks, then their V rows, then the next super-block's K rows,
    // with two blocks' loads (16 KiB) in flight in two register slots: the
    // K-before-V order of §5.6 opt2 (the scores read K first, the softmax
    // and P.V read V later).
    // Measured on MI355X: a wave that streams K and V side by side (two
    // concurrent address streams) gets its bytes later than one that reads
    // them one after the other, and a super-block of two blocks is the
    // largest whose scores fit the registers of three waves per SIMD.
    constexpr int kSblk = 2;
    Slot slot[2];
    // Issues the loads of stream item `it` of super-block q into `dst`; `it`
    // is a compile-time position: 0..kSblk-1 are the K blocks, kSblk ..
    // 2*kSblk-1 the V blocks, and later positions the next super-block's K
    // blocks.  Blocks past the wave's range read zeros (the resources end at
    // its last key), so the loads are unconditional and every wait the
    // compiler inserts is for the one block consumed next.
    auto issue = [&](Slot& dst, int q, int it) __attribute__((always_inline)) {
      const bool isv = it >= kSblk && it < 2 * kSblk;
      const int blk = it < kSblk ? q * kSblk + it
                      : isv      ? q * kSblk + it - kSblk
                                 : (q + 1) * kSblk + it - 2 * kSblk;
      if constexpr (kPaged) {
        __amdgpu_buffer_rsrc_t r[2];
        paged_rsrc(static_cast<const __bf16*>(isv ? p.v : p.k), blk, r);
        if (!isv) {
#pragma unroll
          for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
              dst[4 * sb + kb] = __builtin_amdgcn_raw_buffer_load_b128(r[sb], off.k[0] + 64 * kb, 0, 2);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            dst[j] = __builtin_amdgcn_raw_buffer_load_b128(r[j >> 2], off.v[0] + (j & 3) * kD * 2, 0, 2);
        }
      } else {
        const int boff = blk * (kBlk * kD * 2);
        if (!isv) {
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
            const int vo = off.k[sb] + boff;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
              dst[4 * sb + kb] = __builtin_amdgcn_raw_buffer_load_b128(rk, vo + 64 * kb, 0, 2);
          }
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int vo = off.v[h] + boff;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              dst[4 * h + j] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo + j * kD * 2, 0, 2);
          }
        }
      }
    };
    // Super-blocks that reach past L - T_q hold keys hidden from some rows.
    const int first_hidden = L - p.T_q + 1;
    const int nsb = (nblk + kSblk - 1) / kSblk;
    issue(slot[0], 0, 0);
    issue(slot[1], 0, 1);
    for (int q = 0; q < nsb; ++q) {
      const int key0 = ws + q * kSblk * kBlk;
      // Scores of the super-block; each slot is refilled once read.
      f32x4 s[kSblk][2];
#pragma unroll
      for (int it = 0; it < kSblk; ++it) {
        Slot k;
#pragma unroll
        for (int j = 0; j < 8; ++j) k[j] = slot[it & 1][j];
        block_scores(s[it], k, qb);
        issue(slot[it & 1], q, it + 2);
      }
      // The online-softmax update of §3 over the super-block: one new max,
      // one rescale of l and O.  Keys at or past the wave's end, or past a
      // row's limit `vis_last` (the causal tail of a multi-token decode),
      // get weight 0; only a super-block that holds such keys is masked.
      const int key_end = key0 + kSblk * kBlk;
      const bool masked = key_end > we || key_end > first_hidden;
#pragma unroll
      for (int it = 0; it < kSblk; ++it)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) s[it][sb] *= p.scale_log2;
      if (masked) {
#pragma unroll
        for (int it = 0; it < kSblk; ++it)
#pragma unroll
          for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = key0 + it * kBlk + 16 * sb + 4 * g + i;
              if (key >= we || key > vis_last) s[it][sb][i] = kNegInf;
            }
      }
      float bmax = kNegInf;
#pragma unroll
      for (int it = 0; it < kSblk; ++it)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, s[it][sb][i]);
      bmax = wave_max_xor(bmax, 16);
      bmax = wave_max_xor(bmax, 32);
      const float m_new = fmaxf(st.m, bmax);
      // A row that has seen no visible key yet keeps m = -inf; its weights
      // are taken against 0 (all exp2(-inf) = 0) so that no -inf - -inf appears.
      const float mref = m_new == kNegInf ? 0.f : m_new;
      const float corr = fast_exp2(st.m - mref);  // 0 on a row's first visible keys (m = -inf)
      float psum = 0.f;
      bf16x8 pb[kSblk];   // P^T operands: slots 0..3 = sub-block 0 keys 4g+i, 4..7 = sub-block 1
#pragma unroll
      for (int it = 0; it < kSblk; ++it) {
        float pr[2][4];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pr[sb][i] = fast_exp2(s[it][sb][i] - mref);
            psum += pr[sb][i];
          }
        const u32x4 pw = {pack_bf16x2(pr[0][0], pr[0][1]), pack_bf16x2(pr[0][2], pr[0][3]),
                          pack_bf16x2(pr[1][0], pr[1][1]), pack_bf16x2(pr[1][2], pr[1][3])};
        pb[it] = as_bf16x8(pw);
      }
      st.l = st.l * corr + psum;
      st.m = m_new;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) st.o[dt] *= corr;
      // P.V of the super-block; each slot is refilled once read.
#pragma unroll
      for (int it = kSblk; it < 2 * kSblk; ++it) {
        Slot v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = slot[it & 1][j];
        block_pv(st, v, pb[it - kSblk]);
        issue(slot[it & 1], q, it + 2);
      }
    }
  }

  // Per-query sum over the 4 lane groups that share query n.
  float lsum = wave_sum_xor(st.l, 16);
  lsum = wave_sum_xor(lsum, 32);

  // Merge the 4 waves through LDS.
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];
  __shared__ float sm_o[kWaves][16][kD + 4];
  if (g == 0) {
    sm_m[wave][n] = st.m;
    sm_l[wave][n] = lsum;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int dbase = 8 * (4 * g + i);
    f32x4 lo = {st.o[0][i], st.o[1][i], st.o[2][i], st.o[3][i]};
    f32x4 hi = {st.o[4][i], st.o[5][i], st.o[6][i], st.o[7][i]};
    *reinterpret_cast<f32x4*>(&sm_o[wave][n][dbase]) = lo;
    *reinterpret_cast<f32x4*>(&sm_o[wave][n][dbase + 4]) = hi;
  }
  __syncthreads();

  const size_t part0 = row0 * p.n_split_max + split;
  for (int e = threadIdx.x; e < M * kD; e += blockDim.x) {
    const int qn = e >> 7;
    const int dd = e & (kD - 1);
    float mw[kWaves];
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = sm_m[w][qn];
      M = fmaxf(M, mw[w]);
    }
    float acc = 0.f, lacc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = (mw[w] == kNegInf) ? 0.f : fast_exp2(mw[w] - M);
      acc += wt * sm_o[w][qn][dd];
      lacc += wt * sm_l[w][qn];
    }
    const size_t part = part0 + (size_t)qn * p.n_split_max;
    store_partial(p.ws_o + part * kD + dd, acc, kFused);
    if (dd == 0) {
      store_partial(p.ws_ml + 2 * part, M, kFused);
      store_partial(p.ws_ml + 2 * part + 1, lacc, kFused);
    }
  }
  if constexpr (kFused) fused_merge_tail<__bf16>(p, b, kvh, (L + p.chunk - 1) / p.chunk);
}
}  // namespace

// The two-launch split kernel fits three waves per SIMD (at most 168
// registers); the one-launch kernel, whose merge tail needs more registers,
// is a kernel of its own at two waves per SIMD.  The split kernel takes the
// sequence lengths as its first argument, preloaded into registers (see
// CombineHead): the length load is issued first, together with the loads
// of the other parameters, instead of after them.
template <bool kPaged>
__global__ __launch_bounds__(256, 3) void decode_partial_bf16_kernel(const int32_t* kv_lens, DecodeParams p) {
  const int kv_len = kv_lens[blockIdx.z];
  __builtin_amdgcn_sched_barrier(0);
  decode_partial_bf16<kPaged, false>(p, kv_len);
}

template <bool kPaged>
__global__ __launch_bounds__(256, 2) void decode_fused_bf16_kernel(DecodeParams p) {
  decode_partial_bf16<kPaged, true>(p, p.kv_lens[blockIdx.z]);
}

// fp32 decode partial: one workgroup of 256 threads per 64-key split.  The
// split's K and V rows (32 KiB each) and the group's Q rows are staged in
// LDS with all loads in flight at once; then scores, the split's max and
// sum, and P.V are computed from LDS on the vector ALUs in fp32 (a one-shot
// partial over the split, the "fits in scratch" shape of §5.2).
constexpr int kF32Chunk = 64;

// QS = ceil(G / 4): query slots per thread in the score phase (2*QS in P.V),
// so that no thread computes rows past the group's G heads.
template <int QS>
__global__ __launch_bounds__(256) void decode_partial_f32_kernel(const int32_t* kv_lens, DecodeParams p) {
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  // The sequence lengths come first, preloaded (as for the bf16 kernel).
  const int kv_len = kv_lens[b];
  __builtin_amdgcn_sched_barrier(0);
  const int L = min(kv_len, p.max_kv_len);
  const int start = split * kF32Chunk;
  if (start >= L) return;
  const int cnt = min(kF32Chunk, L - start);
  const int t = threadIdx.x;
  const float* q = static_cast<const float*>(p.q) + ((size_t)b * p.H_q + (size_t)kvh * p.G) * kD;
  const float* kbase = static_cast<const float*>(p.k) + (((size_t)b * p.H_kv + kvh) * p.kv_cap + start) * kD;
  const float* vbase = static_cast<const float*>(p.v) + (((size_t)b * p.H_kv + kvh) * p.kv_cap + start) * kD;

  __shared__ __attribute__((aligned(16))) float sq[16][kD];
  __shared__ float sk[kF32Chunk][kD + 1];   // +1: a wave reading one column of 64 rows hits 64 banks
  __shared__ __attribute__((aligned(16))) float sv[kF32Chunk][kD];
  __shared__ float ss[16][kF32Chunk];
  __shared__ float sm[16], sl[16];

  // Stage Q, K and V.  Rows past the valid length re-read the last valid
  // row; their scores are masked and their V rows are stored as zeros, so
  // the zero weights never meet padding.  Every global load is
  // issued before the first LDS store, so the staging costs one memory
  // round trip.
  constexpr int kTileF4 = kF32Chunk * kD / 4 / 256;   // float4 per thread per tile
  f32x4 qv[2], kv[kTileF4], vv[kTileF4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e4 = t + 256 * i;
    qv[i] = 4 * e4 < p.G * kD ? *reinterpret_cast<const f32x4*>(q + 4 * e4) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < kTileF4; ++i) {
    const int e4 = t + 256 * i;          // float4 index within the tile
    const int row = min(e4 >> 5, cnt - 1), c4 = (e4 & 31) * 4;   // rows past cnt re-read the last
    kv[i] = *reinterpret_cast<const f32x4*>(kbase + (size_t)row * kD + c4);
    vv[i] = *reinterpret_cast<const f32x4*>(vbase + (size_t)row * kD + c4);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e4 = t + 256 * i;
    if (4 * e4 < p.G * kD) *reinterpret_cast<f32x4*>(&sq[0][0] + 4 * e4) = qv[i];
  }
#pragma unroll
  for (int i = 0; i < kTileF4; ++i) {
    const int e4 = t + 256 * i;
    const int row = e4 >> 5, c4 = (e4 & 31) * 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) sk[row][c4 + c] = kv[i][c];
    *reinterpret_cast<f32x4*>(&sv[row][c4]) = row < cnt ? vv[i] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();

  // Scores: thread t -> key j = t % 64, queries t/64, t/64 + 4, ...
  {
    const int j = t & (kF32Chunk - 1);
    const int n0 = t >> 6;
    float acc[QS];
#pragma unroll
    for (int u = 0; u < QS; ++u) acc[u] = 0.f;
#pragma unroll 16
    for (int d = 0; d < kD; ++d) {
      const float kd = sk[j][d];
#pragma unroll
      for (int u = 0; u < QS; ++u) acc[u] = __builtin_fmaf(sq[n0 + 4 * u][d], kd, acc[u]);   // rows >= G unused
    }
#pragma unroll
    for (int u = 0; u < QS; ++u) {
      const int n = n0 + 4 * u;
      if (n < p.G) ss[n][j] = j < cnt ? acc[u] * p.scale_log2 : kNegInf;
    }
  }
  __syncthreads();

  // Max and sum of the split: wave w handles queries w, w + 4, ...; lane =
  // key.
  const int wave = t >> 6, lane = t & 63;
  for (int n = wave; n < p.G; n += 4) {
    float mx = ss[n][lane];
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    const float e = fast_exp2(ss[n][lane] - mx);   // the split has >= 1 valid key
    ss[n][lane] = e;
    float sum = e;
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane == 0) {
      sm[n] = mx;
      sl[n] = sum;
    }
  }
  __syncthreads();

  // O = P . V: thread t -> column d = t % 128, queries t/128 + 2u (all of
  // them in one pass over the keys, one accumulator each).
  const int dd = t & (kD - 1);
  const int n0 = t >> 7;
  const size_t part0 = ((size_t)b * p.H_q + (size_t)kvh * p.G) * p.n_split_max + split;
  float acc[2 * QS];
#pragma unroll
  for (int u = 0; u < 2 * QS; ++u) acc[u] = 0.f;
#pragma unroll 8
  for (int j = 0; j < kF32Chunk; ++j) {
    const float vj = sv[j][dd];
#pragma unroll
    for (int u = 0; u < 2 * QS; ++u) acc[u] = __builtin_fmaf(ss[n0 + 2 * u][j], vj, acc[u]);   // rows >= G unused
  }
#pragma unroll
  for (int u = 0; u < 2 * QS; ++u) {
    const int n = n0 + 2 * u;
    if (n < p.G) {
      const size_t part = part0 + (size_t)n * p.n_split_max;
      const bool fused = p.counters != nullptr;
      store_partial(p.ws_o + part * kD + dd, acc[u], fused);
      if (dd == 0) {
        store_partial(p.ws_ml + 2 * part, sm[n], fused);
        store_partial(p.ws_ml + 2 * part + 1, sl[n], fused);
      }
    }
  }
  if (p.counters != nullptr) fused_merge_tail<float>(p, b, kvh, (L + kF32Chunk - 1) / kF32Chunk);
}


// The combine launch: one wave per (folded row, quarter of d); the values
// its first load round needs come first, preloaded (see CombineHead).
template <typename OutT, int NG>
__global__ __launch_bounds__(64) void decode_combine_kernel(const int32_t* kv_lens, const float* ws_o,
                                                            const float* ws_ml, int n_split_max, int rows_per_seq,
                                                            DecodeParams p) {
  const CombineHead hd{kv_lens, ws_o, ws_ml, n_split_max, rows_per_seq};
  combine_row<OutT, NG>(p, hd, blockIdx.x, blockIdx.y, threadIdx.x);
}

hipError_t launch_decode(const DecodeParams& p, bool bf16, hipStream_t stream, int phases) {
  if (phases & kDecodePartial) {
    dim3 grid(p.n_split_max, p.H_kv, p.B);
    if (bf16) {
      const bool paged = p.block_table != nullptr, fused = p.counters != nullptr;
      if (paged && fused)
        hipLaunchKernelGGL(decode_fused_bf16_kernel<true>, grid, dim3(256), 0, stream, p);
      else if (paged)
        hipLaunchKernelGGL(decode_partial_bf16_kernel<true>, grid, dim3(256), 0, stream, p.kv_lens, p);
      else if (fused)
        hipLaunchKernelGGL(decode_fused_bf16_kernel<false>, grid, dim3(256), 0, stream, p);
      else
        hipLaunchKernelGGL(decode_partial_bf16_kernel<false>, grid, dim3(256), 0, stream, p.kv_lens, p);
    } else {
      switch ((p.G + 3) / 4) {
        case 1: hipLaunchKernelGGL(decode_partial_f32_kernel<1>, grid, dim3(256), 0, stream, p.kv_lens, p); break;
        case 2: hipLaunchKernelGGL(decode_partial_f32_kernel<2>, grid, dim3(256), 0, stream, p.kv_lens, p); break;
        case 3: hipLaunchKernelGGL(decode_partial_f32_kernel<3>, grid, dim3(256), 0, stream, p.kv_lens, p); break;
        default: hipLaunchKernelGGL(decode_partial_f32_kernel<4>, grid, dim3(256), 0, stream, p.kv_lens, p); break;
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // With the fused merge the split kernel writes the outputs itself.
  if ((phases & kDecodeCombine) && p.counters == nullptr) {
    const dim3 grid(p.B * p.H_q * p.T_q, 4);
    const int ng = combine_ng(p.n_split_max);
#define COMBINE_ARGS p.kv_lens, p.ws_o, p.ws_ml, p.n_split_max, p.H_q * p.T_q, p
    if (bf16) {
      if (ng == 2) hipLaunchKernelGGL((decode_combine_kernel<__bf16, 2>), grid, dim3(64), 0, stream, COMBINE_ARGS);
      else if (ng == 4) hipLaunchKernelGGL((decode_combine_kernel<__bf16, 4>), grid, dim3(64), 0, stream, COMBINE_ARGS);
      else hipLaunchKernelGGL((decode_combine_kernel<__bf16, 8>), grid, dim3(64), 0, stream, COMBINE_ARGS);
    } else {
      if (ng == 2) hipLaunchKernelGGL((decode_combine_kernel<float, 2>), grid, dim3(64), 0, stream, COMBINE_ARGS);
      else if (ng == 4) hipLaunchKernelGGL((decode_combine_kernel<float, 4>), grid, dim3(64), 0, stream, COMBINE_ARGS);
      else hipLaunchKernelGGL((decode_combine_kernel<float, 8>), grid, dim3(64), 0, stream, COMBINE_ARGS);
    }
  }
#undef COMBINE_ARGS
  return hipGetLastError();
}

}  // namespace gqa
