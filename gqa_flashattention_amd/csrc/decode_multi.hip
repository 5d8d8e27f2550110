// Multi-token decode for gfx950: T_q new tokens per sequence (speculative or
// short-chunk decode), each attending causally to the cache that already
// holds all T_q of them.  Split-KV partial kernel; the partials are merged
// by the decode combine kernel.
//
// Method: ADR-0060 "AHBM GQA Fused Attention Kernel (Llama3-70B)", revision
// 5a76ed4 -- §3 (running state m, l of shape [G, T_q] and O of [G, T_q, d]:
// the G heads x T_q tokens of one KV head are stacked into the M rows of one
// GEMM, so every K/V tile is streamed once for all of them; additive causal
// mask on boundary tiles only), §5.2 (the same M-fold for decode),
// §0.5.3 (q_block_meta: the block of T_q queries starts at q_start =
// L - T_q, so token t sees keys j <= L - T_q + t) and §4 (unnormalised
// (m, l, O) partials merged by log-sum-exp).
//
// GPU mapping.  One workgroup = W waves = one contiguous split of one
// (sequence, KV head).  The M = G*T_q folded rows (row r = token r % T_q of
// head r / T_q, the memory order of q) form R = 1, 2 or 4 groups of 32;
// wave w takes row group w % R and key slot w / R, so the W waves cover
// R row groups x W/R key slots.  A step stages 32 keys per key slot of K and
// V in LDS (direct global -> LDS loads into a ring of N steps, shared by the
// waves of different row groups) and each wave folds its 32 keys into its
// 32 rows:
//   S^T = K . Q^T on the 32x32x16 bf16 MFMA (keys in M, rows in N), so a
//   lane holds 16 scores of one row (the other 16 sit in lane ^ 32);
//   P = exp2(S*scale - ref) rounded to bf16 is directly the B operand of
//   O^T = V^T . P^T, whose V^T operand comes from the row-major V tile
//   through the transposing LDS read.
// The waves meet at a barrier every step, so they would all run their
// matrix work and their exponentials at the same time; instead each wave
// issues the P.V of step s-1 between the exponentials of step s, keeping
// the matrix unit busy while the vector ALUs work.  V of step s-1 therefore
// stays in LDS through step s and the loads run N-2 steps ahead.
// Softmax statistics use the lazy reference of the prefill kernel: weights
// are taken relative to a per-row reference that moves only when a score
// exceeds it by more than 64 (log2 units), detected by the lane sum of the
// weights; O and l share the reference, so the partial (ref, l, O) is an
// exact (m, l, O) triple for the log-sum-exp merge.  At the end the key
// slots of a row group merge through LDS and one partial per (row, split) is
// written.
//
// Only the last steps of a sequence need the causal tail mask (the T_q - 1
// last keys are not visible to every token); earlier steps run unmasked.

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_tile.hpp"

namespace gqa {

namespace {

constexpr int kD = 128;
constexpr int kSub = 32;               // keys per wave per step
constexpr int kRowBytes = kD * 2;      // one bf16 K or V row

constexpr float kResetGap = 64.f;                       // log2 units
constexpr float kPsumLimit = 18446744073709551616.f;    // 2^64 = exp2(kResetGap)
constexpr float kRefBelow = 32.f;

template <int N>
using Int = std::integral_constant<int, N>;

// f(Int<0>), f(Int<1>), ..., f(Int<N-1>).
template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(Int<I>());
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

// Geometry for R row groups of 32, W waves per workgroup and a ring of N
// steps in LDS.
template <int R, int W, int N>
struct MqShape {
  static constexpr int kWaves = W;
  static constexpr int kThreads = 64 * W;
  static constexpr int kSlots = W / R;                    // key slots
  static constexpr int kStep = kSub * kSlots;             // keys per step
  static constexpr int kStepBytes = kStep * kRowBytes;    // K (or V) bytes of one step
  static constexpr int kRing = N;                         // steps resident in LDS
  static constexpr int kInsts = kStep / 4 / W;            // 1 KiB loads per wave per step, K or V
  static_assert(W % R == 0 && kInsts * 4 * W == kStep, "shape");
  static_assert(2 * N * kStepBytes <= 128 * 1024, "LDS");
  static_assert(N >= 3 && 2 * kInsts * (N - 3) <= 63, "vmcnt");
};

// Launch shape per row-group count: waves per workgroup and ring depth
// (measured on MI355X against 1-8 waves and 3-8 steps; the time barely
// moves, these are the best):
//   R = 1: 2 waves, 64-key steps, 4 steps in LDS (two 32 KiB steps in flight)
//   R = 2: 4 waves, 64-key steps, 4 steps
//   R = 4: 8 waves (two per SIMD), 64-key steps, 4 steps
template <int R> struct MqLaunch;
template <> struct MqLaunch<1> { using S = MqShape<1, 2, 4>; };
template <> struct MqLaunch<2> { using S = MqShape<2, 4, 4>; };
template <> struct MqLaunch<4> { using S = MqShape<4, 8, 4>; };

// s_waitcnt leaving `ahead` (0..A) steps of `kPer` loads each in flight.
template <int kPer, int A>
__device__ __forceinline__ void wait_vm_steps(int ahead) {
  if constexpr (A == 0) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  } else {
    if (ahead >= A) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(A * kPer));
    } else {
      wait_vm_steps<kPer, A - 1>(ahead);
    }
  }
}

// LDS block of one wave's row-group state for the merge of key slots:
// 32 rows x (128 O + m + l + 2 pad) floats.
constexpr int kRedStride = kD + 4;
constexpr int kRedFloats = 32 * kRedStride;

}  // namespace

// Grid: (n_split_max, H_kv, B); block: 64 * W threads.  kPaged: K/V live in
// a page pool addressed through the block table.  What the first loads
// need (the sequence lengths, Q, H_kv and the fold's M = G * T_q rows) comes
// as leading kernel arguments, which this file's build preloads into
// registers: the length and Q loads issue at wave start, before the
// argument block has arrived.
template <int R, bool kPaged>
__global__ __launch_bounds__(MqLaunch<R>::S::kThreads, 1) void decode_multi_partial_kernel(
    const int32_t* kv_lens, const __bf16* q, int H_kv, int M, DecodeParams p) {
  using S = typename MqLaunch<R>::S;
  // K ring then V ring, contiguous so that the merge can reuse both.
  __shared__ __attribute__((aligned(1024))) __bf16 sKV[2][S::kRing][S::kStep * kD];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int rg = wave % R;      // row group
  const int kq = wave / R;      // key slot
  const int c = lane & 31;      // row of this lane within the row group
  const int h2 = lane >> 5;
  const int t16 = lane & 15;
  const int gamma = lane >> 4;

  const int row = 32 * rg + c;
  const bool row_ok = row < M;
  const size_t row0 = ((size_t)b * H_kv + kvh) * M;   // first folded row: (b*H_q + kvh*G)*T_q

  // Q^T operand (B of S^T): row `row`, d = 16*kk + 8*h2 .. +8, through a
  // buffer resource that ends at the M-th folded row, so that padding rows
  // read as zeros without a branch.  These loads do not depend on the
  // sequence length and are issued together with its load, so the two
  // round trips overlap; a negative scale is applied exactly below by
  // flipping Q's sign bits.
  const int kv_len = kv_lens[b];
  u32x4 qv[8];
  {
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(q + row0 * kD), (short)0, (unsigned)M * kRowBytes, 0x00020000);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qv[kk] = __builtin_amdgcn_raw_buffer_load_b128(rq, row * kRowBytes + 16 * h2 + 32 * kk, 0, 0);
  }
  // Nothing that reads the argument block is scheduled above these loads.
  __builtin_amdgcn_sched_barrier(0);
  const int start = split * p.chunk;
  // Paged: lanes j and 64 + j fetch the block-table entries of the split's
  // logical pages lp0 + j and lp0 + 64 + j (at most 128 pages per split,
  // checked on the host).  The split's first page follows from the split
  // alone, so these loads are issued together with the sequence length's;
  // entries past the table row are clamped to its last one, and those past
  // the sequence are not used.
  const int shift = p.page_shift;
  const int lp0 = start >> shift;
  int pt_raw[2] = {0, 0};
  if constexpr (kPaged) {
    const int32_t* trow = p.block_table + (size_t)b * p.max_pages;
    const int j = threadIdx.x & 63;
    pt_raw[0] = trow[min(lp0 + j, p.max_pages - 1)];
    pt_raw[1] = trow[min(lp0 + 64 + j, p.max_pages - 1)];
  }
  const int L = min(kv_len, p.max_kv_len);
  // Keeps these loads above the early exit below (the compiler would
  // otherwise sink them there, behind the length's round trip).  Q is
  // complete from here on, before any of the ring's direct-to-LDS loads is
  // issued: the compiler does not count those, so a later first use of Q
  // would wait for them too.
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) asm volatile("" : "+v"(qv[kk]));
  if constexpr (kPaged) asm volatile("" : "+v"(pt_raw[0]), "+v"(pt_raw[1]));
  if (start >= L) return;
  const int end = min(start + p.chunk, L);
  const int nsteps = (end - start + S::kStep - 1) / S::kStep;
  // Steps [0, n_full) hold only keys every row sees (keys below L - T_q + 1).
  const int n_full = max(0, min(L - p.T_q + 1, end) - start) / S::kStep;
  // Last key this lane's row may see within the split (padding rows see all).
  const int vis_last = row_ok ? min(L - p.T_q + row % p.T_q, end - 1) : end - 1;

  const __bf16* Kg = static_cast<const __bf16*>(p.k) + (kPaged ? 0 : ((size_t)b * p.H_kv + kvh) * p.kv_cap * kD);
  const __bf16* Vg = static_cast<const __bf16*>(p.v) + (kPaged ? 0 : ((size_t)b * p.H_kv + kvh) * p.kv_cap * kD);

  bf16x8 qb[8];
  {
    const unsigned flip = p.q_negate ? 0x80008000u : 0u;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qb[kk] = as_bf16x8(qv[kk] ^ u32x4{flip, flip, flip, flip});
  }

  // Per-lane LDS addresses of the MFMA operands in ring slot 0 (other slots
  // are immediate offsets), hidden from the compiler so that it keeps the
  // offsets in the instructions.
  //  K (A of S^T), k-step kk: row 32*kq + c, logical piece 2*kk + h2.
  //  V (A of O^T, transposing read), key step st, d-tile dt: rows
  //    32*kq + 16*st + 4*h2 + t16/4 and 8 rows further, d = 32*dt +
  //    16*(gamma&1) + 4*(t16&3) .. +4; the lane receives V^T column
  //    d = 32*dt + 16*(gamma&1) + t16.
  const unsigned lds_k0 = lds_addr(&sKV[0][0][0]);
  const unsigned lds_v0 = lds_addr(&sKV[1][0][0]);
  unsigned kaddr[8], vaddr[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    kaddr[kk] = lds_k0 + (32 * kq + c) * kRowBytes + 16 * k_swz(c, 2 * kk + h2);
    asm volatile("" : "+v"(kaddr[kk]));
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int r0 = 32 * kq + 4 * h2 + (t16 >> 2);
    const int e = 32 * dt + 16 * (gamma & 1) + 4 * (t16 & 3);
    vaddr[dt] = lds_v0 + r0 * kRowBytes + 16 * v_swz(r0, e >> 3) + 2 * (e & 7);
    asm volatile("" : "+v"(vaddr[dt]));
  }

  // Direct global -> LDS loads of one step: the waves split the step's row
  // groups of 4; lane l lands at physical piece l%16 of row 4*group + l/16
  // and fetches the logical piece that belongs there.  The buffer resource
  // ends at the split's last key, so rows past it read as zeros (masked,
  // with zero V rows) and nothing outside the split is read.
  int ld_off[2][S::kInsts];
#pragma unroll
  for (int i = 0; i < S::kInsts; ++i) {
    const int r = 4 * (S::kInsts * wave + i) + (lane >> 4);
    ld_off[0][i] = r * kRowBytes + 16 * k_swz(r, lane & 15);   // XOR is an involution
    ld_off[1][i] = r * kRowBytes + 16 * v_swz(r, lane & 15);
  }
  // Paged: lane j of pt[0] / pt[1] holds the physical page of the split's
  // logical page lp0 + j / lp0 + 64 + j (at most 128 pages per split,
  // checked on the host); entries are clamped into the pool.
  int pt[2] = {0, 0};
  if constexpr (kPaged) {
    const int npg = ((end - 1) >> shift) - lp0 + 1;
    if (lane < npg) pt[0] = min(max(pt_raw[0], 0), p.num_pages - 1);
    if (lane + 64 < npg) pt[1] = min(max(pt_raw[1], 0), p.num_pages - 1);
  }
  auto load_step = [&](auto slot_c, int s) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    const int key0 = start + s * S::kStep;
    if constexpr (kPaged) {
      // One resource per 1 KiB instruction (4 rows, always inside one page):
      // based so that the instruction's lane offsets land on its rows, and
      // ending at the split's last key (rows past it read as zeros).
      const size_t page_elems = (size_t)p.H_kv * (kD << shift);
      const size_t head_elems = (size_t)kvh * (kD << shift);
#pragma unroll
      for (int i = 0; i < S::kInsts; ++i) {
        const int r0 = 4 * (S::kInsts * wave + i);
        const int pos = key0 + r0;
        const int idx = min((pos >> shift) - lp0, 127);
        const int pp = idx < 64 ? __builtin_amdgcn_readlane(pt[0], idx)
                                : __builtin_amdgcn_readlane(pt[1], idx - 64);
        const size_t e = (size_t)pp * page_elems + head_elems + (size_t)(pos & ((1 << shift) - 1)) * kD;
        const unsigned nb = (unsigned)(r0 + max(0, min(4, end - pos))) * kRowBytes;
        const uintptr_t kb = reinterpret_cast<uintptr_t>(static_cast<const __bf16*>(p.k) + e) - (uintptr_t)r0 * kRowBytes;
        const uintptr_t vb = reinterpret_cast<uintptr_t>(static_cast<const __bf16*>(p.v) + e) - (uintptr_t)r0 * kRowBytes;
        dma_load_x4(ld_off[0][i], buffer_rsrc(reinterpret_cast<const void*>(kb), nb),
                    lds_k0 + slot * S::kStepBytes + 4 * (S::kInsts * wave + i) * kRowBytes);
        dma_load_x4(ld_off[1][i], buffer_rsrc(reinterpret_cast<const void*>(vb), nb),
                    lds_v0 + slot * S::kStepBytes + 4 * (S::kInsts * wave + i) * kRowBytes);
      }
    } else {
      const unsigned bytes = (unsigned)(end - key0) * kRowBytes;
      const u32x4 rk = buffer_rsrc(Kg + (size_t)key0 * kD, bytes);
      const u32x4 rv = buffer_rsrc(Vg + (size_t)key0 * kD, bytes);
#pragma unroll
      for (int i = 0; i < S::kInsts; ++i)
        dma_load_x4(ld_off[0][i], rk, lds_k0 + slot * S::kStepBytes + 4 * (S::kInsts * wave + i) * kRowBytes);
#pragma unroll
      for (int i = 0; i < S::kInsts; ++i)
        dma_load_x4(ld_off[1][i], rv, lds_v0 + slot * S::kStepBytes + 4 * (S::kInsts * wave + i) * kRowBytes);
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m_ref = kNegInf;   // reference (log2 units) of this lane's row, same on both halves
  float lpart = 0.f;       // this lane's half of the running sum, relative to m_ref
  // |scale| * log2(e), kept away from zero so that masked (-inf) scores
  // stay -inf.
  const float sl2 = fmaxf(p.scale_log2, 1e-30f);

  // P = exp2(S*scale - ref) of the lane's 16 scores, rounded to bf16 in the
  // P^T operand layout (key step st: keys 16*st + {0..3, 8..11} + 4*h2);
  // returns their fp32 sum.
  auto exps = [&](const f32x16& sacc, float negr, u32x4 (&pw)[2]) __attribute__((always_inline)) -> float {
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float e0 = fast_exp2(__builtin_fmaf(sacc[8 * st + 2 * jj], sl2, negr));
        const float e1 = fast_exp2(__builtin_fmaf(sacc[8 * st + 2 * jj + 1], sl2, negr));
        psum += e0 + e1;
        pw[st][jj] = pack_bf16x2(e0, e1);
      }
    return psum;
  };

  // O^T += V^T . P^T of one step from ring slot `slot` (8 MFMAs).  The V
  // operand reads are issued first, then the MFMAs.
  auto pv_reads = [&](auto slot_c, bf16x8 (&va)[8]) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const unsigned a = vaddr[dt] + slot * S::kStepBytes + 4096 * st;
        const u32x2 w0 = __builtin_bit_cast(u32x2, lds_read_tr16(a));
        const u32x2 w1 = __builtin_bit_cast(u32x2, lds_read_tr16(a + 8 * kRowBytes));
        const u32x4 av = {w0[0], w0[1], w1[0], w1[1]};
        va[4 * st + dt] = as_bf16x8(av);
      }
  };

  // Step s: scores of this wave's 32 keys against its 32 rows (S MFMAs),
  // the tail mask (last steps only), then the softmax of step s issued
  // between the 8 MFMAs of the previous step's P.V (`pprev`, V from slot
  // `pslot`), so that the matrix unit works while the vector ALUs compute
  // the exponentials.  P of step s is left in `pprev` for the next step.
  u32x4 pprev[2] = {u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}};
  auto compute = [&](auto slot_c, auto pslot_c, int s) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    // All eight K operand reads are issued before the first MFMA (one LDS
    // round trip per step instead of eight).
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 ka[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) ka[kk] = *lds_ptr<bf16x8>(kaddr[kk] + slot * S::kStepBytes);
    f32x16 sacc;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const f32x16 zero = {};
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qb[kk], kk ? sacc : zero, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // the 8 K reads
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // then the 8 S MFMAs
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 va[8];
    pv_reads(pslot_c, va);
    if (s >= n_full) {
      const int key0 = start + s * S::kStep + 32 * kq;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + 8 * (i >> 2) + 4 * h2 + (i & 3);
        if (key > vis_last) sacc[i] = kNegInf;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // Softmax of step s against the reference, one exponential pair per
    // P.V MFMA of step s-1.
    const float negr = -m_ref;
    u32x4 pw[2];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], as_bf16x8(pprev[i >> 2]), o[i & 3],
                                                         0, 0, 0);
      const int st = i >> 2, jj = i & 3;
      const float e0 = fast_exp2(__builtin_fmaf(sacc[8 * st + 2 * jj], sl2, negr));
      const float e1 = fast_exp2(__builtin_fmaf(sacc[8 * st + 2 * jj + 1], sl2, negr));
      psum += e0 + e1;
      pw[st][jj] = pack_bf16x2(e0, e1);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // then the pair's VALU work
    }
    __builtin_amdgcn_sched_barrier(0);
    if (__any(!(psum <= kPsumLimit))) {
      // Some weight exceeds 2^64 (a score more than 64 above the reference,
      // always so on a row's first visible keys): move the reference of
      // such rows to 32 below their max, rescale O (which now holds steps
      // up to s-1) and l, redo P.  A row with no visible key yet keeps the
      // reference -inf and gets P = 0.
      float hmax = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) hmax = fmaxf(hmax, sacc[i]);
      const float rmax = wave_max_xor(hmax, 32) * sl2;
      const float m_new = rmax > m_ref + kResetGap ? rmax - kRefBelow : m_ref;
      const float corr = m_new == m_ref ? 1.f : fast_exp2(m_ref - m_new);
      lpart *= corr;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= corr;
      m_ref = m_new;
      psum = exps(sacc, m_ref == kNegInf ? 0.f : -m_ref, pw);
    }
    lpart += psum;
    pprev[0] = pw[0];
    pprev[1] = pw[1];
  };

  // Ring schedule.  Step s reads K of step s and V of step s-1, so slot
  // (s-1) % N is free only after step s; the loads run N-2 steps ahead.
  // Steps 0 .. N-3 are loaded up front.  Step s waits for its own loads
  // (leaving the later steps' loads in flight), meets the other waves at a
  // barrier (their loads of step s have landed, and all are done with step
  // s-1, the last reader of slot (s-2) % N), issues the load of step
  // s + N - 2 into that slot and computes.  The first step's P.V reads the
  // V slot N-1 with P = 0; that slot is zeroed so that no stale bit pattern
  // (a NaN) meets the zero weights.
  constexpr int kPer = 2 * S::kInsts;   // load instructions per wave per step
  auto wait_step = [&](int s) __attribute__((always_inline)) {
    const int ahead = min(S::kRing - 3, nsteps - 1 - s);   // later steps already issued
    wait_vm_steps<kPer, S::kRing - 3>(ahead);
  };
  auto step = [&](auto slot_c, int s) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    wait_step(s);
    __syncthreads();
    if (s + S::kRing - 2 < nsteps) load_step(Int<(slot + S::kRing - 2) % S::kRing>(), s + S::kRing - 2);
    compute(slot_c, Int<(slot + S::kRing - 1) % S::kRing>(), s);
  };

  {
    u32x4* z = reinterpret_cast<u32x4*>(&sKV[1][S::kRing - 1][0]);
    for (int i = t; i < S::kStep * kD / 8; i += S::kThreads) z[i] = u32x4{0, 0, 0, 0};
  }
  // Prologue loads, then the steps in groups of N so that ring slots are
  // compile-time constants, then the remaining steps, then the last P.V.
  static_for<S::kRing - 2>([&](auto i_c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    if (i < nsteps) load_step(Int<i>(), i);
  });
  int s = 0;
  for (; s + S::kRing <= nsteps; s += S::kRing) {
    static_for<S::kRing>([&](auto i_c) __attribute__((always_inline)) {
      step(i_c, s + decltype(i_c)::value);
    });
  }
  static_for<S::kRing - 1>([&](auto i_c) __attribute__((always_inline)) {
    if (s + decltype(i_c)::value < nsteps) step(i_c, s + decltype(i_c)::value);
  });
  {
    // P.V of the last step, whose V is in slot (nsteps - 1) % N.
    const int last = (nsteps - 1) % S::kRing;
    static_for<S::kRing>([&](auto i_c) __attribute__((always_inline)) {
      if (decltype(i_c)::value == last) {
        bf16x8 va[8];
        pv_reads(i_c, va);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], as_bf16x8(pprev[i >> 2]),
                                                             o[i & 3], 0, 0, 0);
      }
    });
  }

  // Row sums over both halves; merge the key slots of each row group.
  const float lrow = lpart + __shfl_xor(lpart, 32, 64);
  float m_out = m_ref, l_out = lrow;
  if constexpr (S::kSlots > 1) {
    float* red = reinterpret_cast<float*>(&sKV[0][0][0]);
    static_assert((S::kSlots - 1) * R * kRedFloats * 4 <= (int)sizeof(sKV), "merge buffer");
    __syncthreads();   // all waves are done with the ring (every load was waited for)
    if (kq > 0) {
      float* mine = red + ((kq - 1) * R + rg) * kRedFloats + c * kRedStride;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 v = {o[dt][4 * i4], o[dt][4 * i4 + 1], o[dt][4 * i4 + 2], o[dt][4 * i4 + 3]};
          *reinterpret_cast<f32x4*>(mine + 32 * dt + 8 * i4 + 4 * h2) = v;
        }
      if (h2 == 0) {
        mine[kD] = m_ref;
        mine[kD + 1] = lrow;
      }
    }
    __syncthreads();
    if (kq > 0) return;
    float mk[S::kSlots];
    mk[0] = m_ref;
    float mmax = m_ref;
#pragma unroll
    for (int k = 1; k < S::kSlots; ++k) {
      mk[k] = red[((k - 1) * R + rg) * kRedFloats + c * kRedStride + kD];
      mmax = fmaxf(mmax, mk[k]);
    }
    const float w0 = mk[0] == kNegInf ? 0.f : fast_exp2(mk[0] - mmax);
    l_out = lrow * w0;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= w0;
#pragma unroll
    for (int k = 1; k < S::kSlots; ++k) {
      const float* other = red + ((k - 1) * R + rg) * kRedFloats + c * kRedStride;
      const float wk = mk[k] == kNegInf ? 0.f : fast_exp2(mk[k] - mmax);
      l_out += wk * other[kD + 1];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(other + 32 * dt + 8 * i4 + 4 * h2);
#pragma unroll
          for (int u = 0; u < 4; ++u) o[dt][4 * i4 + u] += wk * v[u];
        }
    }
    m_out = mmax;
  }

  // The partial of (row, split): O in the lane's d = 32*dt + 8*i4 + 4*h2
  // .. +4, and (m, l) from the first half.
  if (row_ok) {
    const size_t part = (row0 + row) * p.n_split_max + split;
    float* wo = p.ws_o + part * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 v = {o[dt][4 * i4], o[dt][4 * i4 + 1], o[dt][4 * i4 + 2], o[dt][4 * i4 + 3]};
        *reinterpret_cast<f32x4*>(wo + 32 * dt + 8 * i4 + 4 * h2) = v;
      }
    if (h2 == 0) {
      p.ws_ml[2 * part] = m_out;
      p.ws_ml[2 * part + 1] = l_out;
    }
  }
}

int decode_multi_row_groups(int M) { return M <= 32 ? 1 : (M <= 64 ? 2 : 4); }

hipError_t launch_decode_multi(const DecodeParams& p, hipStream_t stream, int phases) {
  if (phases & kDecodePartial) {
    const dim3 grid(p.n_split_max, p.H_kv, p.B);
    const bool paged = p.block_table != nullptr;
#define MULTI_ARGS p.kv_lens, static_cast<const __bf16*>(p.q), p.H_kv, p.G * p.T_q, p
    switch (decode_multi_row_groups(p.G * p.T_q)) {
      case 1:
        if (paged)
          hipLaunchKernelGGL((decode_multi_partial_kernel<1, true>), grid, dim3(MqLaunch<1>::S::kThreads), 0, stream,
                             MULTI_ARGS);
        else
          hipLaunchKernelGGL((decode_multi_partial_kernel<1, false>), grid, dim3(MqLaunch<1>::S::kThreads), 0, stream,
                             MULTI_ARGS);
        break;
      case 2:
        if (paged)
          hipLaunchKernelGGL((decode_multi_partial_kernel<2, true>), grid, dim3(MqLaunch<2>::S::kThreads), 0, stream,
                             MULTI_ARGS);
        else
          hipLaunchKernelGGL((decode_multi_partial_kernel<2, false>), grid, dim3(MqLaunch<2>::S::kThreads), 0, stream,
                             MULTI_ARGS);
        break;
      default:
        if (paged)
          hipLaunchKernelGGL((decode_multi_partial_kernel<4, true>), grid, dim3(MqLaunch<4>::S::kThreads), 0, stream,
                             MULTI_ARGS);
        else
          hipLaunchKernelGGL((decode_multi_partial_kernel<4, false>), grid, dim3(MqLaunch<4>::S::kThreads), 0, stream,
                             MULTI_ARGS);
        break;
    }
#undef MULTI_ARGS
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & kDecodeCombine) return launch_decode(p, true, stream, kDecodeCombine);
  return hipSuccess;
}

}  // namespace gqa
