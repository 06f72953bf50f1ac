// attn_fwd_bf16_pp.hip -- the fused attention forward for gfx950, bf16 in / bf16 out,
// 8-wave "ping-pong" workgroups (head dimension 128, grids that fill the GPU).
//
// One kernel computes O = softmax(Q K^T * scale + mask) V and the LSE.  The score
// tile, its row maximum and sum, the exponentials, the online correction
// exp(m_old - m_new) and the P.V product never leave the workgroup (page
// "Attention softmax fusion", sections "What fused has to mean" and "The tile
// loop"; page "Kernel Fusion and the Memory Wall", section "FlashAttention: avoid
// the full score matrix").
//
// Work split.  One workgroup = 8 waves = 256 query rows of one (batch, head); each
// wave owns 32 rows for the whole key loop, and all 8 waves share each 64-key K/V
// tile in LDS.  Waves w and w+4 run on the same SIMD.  They form two groups,
// G0 = waves 0-3 and G1 = waves 4-7, that run the same loop half a tile apart
// ("ping-pong"): while one group issues its matrix instructions (P.V of the
// previous tile and Q.K^T of this one), the other computes its softmax on the
// vector ALU.  A workgroup barrier between phases keeps the two groups in step, so
// the matrix cores of every SIMD see one group's MFMA stream at all times and the
// vector work of the other group hides behind it.
//
//   phase   G0                          G1
//   0       S(0) = K(0) Q^T             -
//   1       softmax(0) -> P(0)          S(0)
//   2       O += V(0) P(0); S(1)        softmax(0)
//   3       softmax(1)                  O += V(0) P(0); S(1)
//   ...     (every phase ends with a workgroup barrier)
//
// Register and LDS layouts (transposed scores, P straight from the score registers,
// swizzled K and V tiles) and the lazy online correction are described in
// attn_bf16_tiles.hpp.
//
// Masking.  The leading key tiles that every row of the workgroup sees whole run a
// copy of the loop body with no mask code and no mask test; only the tiles at the
// causal diagonal or the key-length tail take the body that checks, per wave, whether
// the tile needs masking.  Scalar control flow in the softmax phase is not free: this
// split alone is worth about 2 % at B=1 H=32 N=8192 D=128, causal.  On those boundary
// tiles a wave none of whose rows sees any key of the tile (the causal diagonal block,
// the key-length tail) skips that tile's products and softmax, whose contributions
// would be exact zeros; it still moves data and meets every barrier.
//
// Data movement.  Both tiles go from global memory straight into LDS (buffer_load
// ... lds, no staging registers), row-major, double buffered.  G0 moves all of it:
// in its matrix phase of tile t (the first phase after the last reads of those
// buffers) it requests V(t) and K(t+1), spread between its MFMAs, and it waits for
// them at the end of its softmax phase, before the barrier that publishes them.  (A
// wave whose request the memory pipeline cannot take yet stalls; in a matrix phase
// the matrix core works through its queued MFMAs meanwhile, in a softmax phase the
// exponentials would wait.)  The 16-byte chunks of a row are XOR-swizzled with a
// function of the row (kswz for K, vswz for V), so the fragment reads are bank-conflict
// free: K fragments by ds_read_b128, the P.V operand (8 consecutive keys of one
// dimension) by two transposing ds_read_b64_tr_b16.  Each buffer is an LDS array of
// its own (see the declarations below).  Buffer indices are compile-time constants
// (the loop is unrolled by two), so every fragment address is a per-lane register
// computed once plus an immediate offset.

#include <type_traits>

#include "attn_bf16_tiles.hpp"
#include "launch.hpp"

namespace attn89 {
namespace {

constexpr int kXcds = 8;   // XCDs of an MI355X

template <int D>
struct Cfg {
  static constexpr int BR = 256;                 // query rows per workgroup
  static constexpr int BC = 64;                  // keys per tile
  static constexpr int NT = 512;                 // threads per workgroup (8 waves)
  static constexpr int ROWB = D * 2;             // bytes per K row
  static constexpr int TILE = BC * ROWB;         // bytes per K (or V) tile
  static constexpr int KDMA = TILE / 1024 / 4;   // 1 KiB loads per wave per tile
  static constexpr int DSTEPS = D / 16;          // k-steps of S^T = K Q^T
  static constexpr int DBLK = D / 32;            // 32-dimension blocks of O^T
  static constexpr int KBLK = BC / 32;           // 32-key blocks of a tile
};

// Phase boundary: this wave's LDS accesses are complete, then all 8 waves meet.
// Outstanding global loads into registers stay in flight (a plain __syncthreads
// would also wait for them).
__device__ __forceinline__ void phase_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Instruction order of an MFMA phase with NR fragment reads and NR MFMAs: kPrefetch
// reads first, then one read after every MFMA, so each fragment is requested
// kPrefetch MFMAs (kPrefetch x 32 cycles) before it is needed.  Left to itself the
// compiler issues each read just before its MFMA and the matrix core waits out the
// LDS latency every time.
constexpr int kPrefetch = 4;
template <int NR>
__device__ __forceinline__ void schedule_mfma_phase() {
  __builtin_amdgcn_sched_group_barrier(0x100, kPrefetch, 0);   // LDS reads
#pragma unroll
  for (int i = 0; i < NR - kPrefetch; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // one LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kPrefetch, 0);
}

// The same for MFMAs that take two fragment reads each (P.V operands gathered by
// transposing reads), optionally followed by NQ MFMAs with one read each (Q.K^T).
// NVM global-memory requests (tile DMA) go one after every kVmStride MFMAs: the memory
// pipeline accepts a CU's requests at a limited rate, and a wave whose request has to
// wait stalls, which costs little while the matrix core still has queued MFMAs.
constexpr int kVmStride = 2;
template <int NPV, int NQ, int NVM = 0>
__device__ __forceinline__ void schedule_mfma_phase_pv() {
  static_assert(NVM <= (NPV + NQ - kPrefetch) / kVmStride, "room for every request");
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPrefetch, 0);
#pragma unroll
  for (int i = 0; i < NPV + NQ - kPrefetch; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < NPV - kPrefetch)
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    else
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (i % kVmStride == kVmStride - 1 && i / kVmStride < NVM)
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kPrefetch, 0);
}

// The wave in its MFMA phase gets issue priority over its SIMD partner (which is in
// its softmax phase), so the matrix core is refilled as soon as it frees up.
__device__ __forceinline__ void mfma_priority() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void valu_priority() { __builtin_amdgcn_s_setprio(0); }

// PRE: scale <= 0, so scores are scaled before they are masked (a separate
// instantiation keeps that branch out of the common kernel).
template <int D, bool PRE>
__global__ __launch_bounds__(512) void attn_fwd_bf16_pp_kernel(FwdArgs p) {
  using C = Cfg<D>;
  // K and V double buffers, each buffer an LDS array of its own, so the compiler can
  // tell that a fragment read of one buffer does not touch another one while a DMA
  // into it is in flight (for reads it cannot separate from a pending DMA target it
  // waits for every outstanding load first)
  __shared__ __attribute__((aligned(1024))) unsigned char smem_k0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char smem_k1[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char smem_v0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char smem_v1[C::TILE];
  auto kbuf = [&](int buf) __attribute__((always_inline)) {
    return buf ? (lds_u8*)smem_k1 : (lds_u8*)smem_k0;
  };
  auto vbuf = [&](int buf) __attribute__((always_inline)) {
    return buf ? (lds_u8*)smem_v1 : (lds_u8*)smem_v0;
  };

  const int tid = threadIdx.x;
  // wave-uniform values live in scalar registers, so branches on them are real
  // branches (a barrier must never sit in a lane-masked region)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;     // 0: G0 (moves K and V), 1: G1
  const int wg = wave & 3;       // wave inside its group
  const int lane = tid & 63;
  const int lq = lane & 31;      // query column inside the wave's 32 rows
  const int lg = lane >> 5;      // half of the wave

  // Schedule.  Workgroups are dispatched to the 8 XCDs round robin (workgroup i runs
  // on XCD i mod 8), so when B*H is a multiple of 8 every query block of a head lands
  // on one XCD and its K/V re-reads can stay in that XCD's L2.
  //  * non-causal: every block of a head has the same length, and each XCD takes its
  //    heads one at a time (all query blocks of one head, then the next), so the K/V
  //    of only a few heads is live in its L2 at once;
  //  * causal, B*H a multiple of 16: each XCD takes its heads two at a time, the
  //    blocks of the two interleaved and heaviest (last) first.  The blocks of a head
  //    differ in length; when the first ones finish, the CUs that ran short blocks take
  //    the long ones that remain, so every CU ends with the same number of key tiles,
  //    and the blocks that run together share their K/V tiles in L2 (taking an XCD's
  //    heads four at a time read 1.7 times as much from device memory; one at a time
  //    read the least but ran slower);
  //  * otherwise consecutive workgroups take different (b, h) of the same query block,
  //    heaviest blocks first.
  const int BH = p.B * p.H;
  const int n_qb = (p.Nq + C::BR - 1) / C::BR;
  int qb, bh;
  if (!p.causal && BH % kXcds == 0) {
    const int x = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
    bh = x + kXcds * (slot / n_qb);
    qb = n_qb - 1 - slot % n_qb;
  } else if (BH % (2 * kXcds) == 0) {
    // (a branch of its own: the same formula merged into the one above makes the
    // compiler spill in the key loop)
    const int x = (int)blockIdx.x & (kXcds - 1), slot = (int)blockIdx.x >> 3;
    const int pair = slot / (2 * n_qb), r = slot - pair * 2 * n_qb;
    bh = x + kXcds * (2 * pair + (r & 1));
    qb = n_qb - 1 - (r >> 1);
  } else {
    qb = n_qb - 1 - (int)blockIdx.x / BH;
    bh = (int)blockIdx.x % BH;
  }
  const int b = bh / p.H;

  const unsigned short* qp = (const unsigned short*)p.q + (size_t)bh * p.Nq * D;
  const unsigned short* kp = (const unsigned short*)p.k + (size_t)bh * p.Nk * D;
  const unsigned short* vp = (const unsigned short*)p.v + (size_t)bh * p.Nk * D;
  unsigned short* op = (unsigned short*)p.o + (size_t)bh * p.Nq * D;
  float* lsep = p.lse + (size_t)bh * p.Nq;

  const int L = clamp_len(p.kv_lens, b, p.Nk);      // valid keys of this sequence
  const int q0 = qb * C::BR;
  const int q_hi = min(q0 + C::BR, p.Nq);
  const int kv_end = p.causal ? min(L, q_hi) : L;    // keys any row of the block sees
  const int n_tiles = (kv_end + C::BC - 1) / C::BC;
  // leading tiles whose keys are all visible to every row of the block
  const int n_full = PRE ? 0 : min(L, p.causal ? q0 + 1 : L) / C::BC;
  const int qw = q0 + wave * 32;                     // first row of this wave
  const int qrow = qw + lq;

  // ---- Q fragments (B operand of S^T = K Q^T), resident for the whole loop ----
  // Buffer loads: rows past Nq (and below, keys past kv_len) read as zeros.
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qp, (unsigned)p.Nq * D * 2);
  bf16x8 qf[C::DSTEPS];
#pragma unroll
  for (int s = 0; s < C::DSTEPS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8,
                               buffer_load16(qrs, ((unsigned)qrow * D + 16 * s + 8 * lg) * 2));

  // ---- K (G0): global -> LDS without registers ----
  // Load n of G0 wave wg writes tile bytes [m*1024, m*1024 + 1024), m = wg*KDMA + n,
  // lane i the 16 bytes at m*1024 + 16*i; the lane fetches the global chunk the
  // swizzle puts there.  The tile start is the scalar offset of the load.
  // Keys from kv_end on (which no row of the block sees) read as zeros, so the request
  // for the tile past the last one fetches nothing.
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (unsigned)kv_end * D * 2);
  unsigned koff[C::KDMA];
#pragma unroll
  for (int n = 0; n < C::KDMA; ++n) {
    const int byte = (wg * C::KDMA + n) * 1024 + 16 * lane;
    const int row = byte / C::ROWB;
    const int ch = ((byte % C::ROWB) / 16) ^ kswz<D>(row);
    koff[n] = ((unsigned)row * D + 8 * ch) * 2;
  }
  auto load_k = [&](int t, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < C::KDMA; ++n)
      buffer_load16_to_lds(krs, (lds_void*)(kbuf(stage) + (wg * C::KDMA + n) * 1024),
                           koff[n], t * C::BC * D * 2);
  };

  // ---- V (G0): global -> LDS without registers, row-major ----
  // Same movement as K, with the V swizzle vswz (row bits 0-1 pick the 64-byte window).
  // The P.V operand (one dimension per lane, the 8 keys of its P fragment) is read back
  // with the transposing ds_read_b64_tr_b16 (see lds_tr16): the lane at position
  // i = 4m + a of a group of 16 lanes (group g) addresses, in read q, key
  // 8(g/2) + 4q + m (plus the P.V step's 16-key offset) at dimensions
  // 16(g%2) + 4a .. + 4 of the 32-dimension block, so two reads give a lane its 8
  // elements; the four keys one read gathers fall in four different 64-byte windows.
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, (unsigned)L * D * 2);
  unsigned voff[C::KDMA];
#pragma unroll
  for (int n = 0; n < C::KDMA; ++n) {
    const int byte = (wg * C::KDMA + n) * 1024 + 16 * lane;
    const int row = byte / C::ROWB;
    const int ch = ((byte % C::ROWB) / 16) ^ vswz<D>(row);
    voff[n] = ((unsigned)row * D + 8 * ch) * 2;
  }
  auto load_v = [&](int t, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < C::KDMA; ++n)
      buffer_load16_to_lds(vrs,
                           (lds_void*)(vbuf(stage) + (wg * C::KDMA + n) * 1024),
                           voff[n], t * C::BC * D * 2);
  };
  unsigned vtr[C::DBLK];   // read q of 32-dimension block d at P.V step s: + (16 s + 4 q) rows
  {
    const int gi = lane & 15, gg = lane >> 4, a = gi & 3, m = gi >> 2;
    const int key = 8 * (gg >> 1) + m;
#pragma unroll
    for (int d = 0; d < C::DBLK; ++d)
      vtr[d] = key * C::ROWB + (((4 * d + 2 * (gg & 1) + (a >> 1)) ^ vswz<D>(key)) * 16) +
               8 * (a & 1);
  }

  // ---- fragment read offsets (per lane, fixed for the whole loop) ----
  const int krow = swap_bits23(lq);   // key (row of K) this lane feeds to the MFMA
  unsigned kro[C::DSTEPS];
#pragma unroll
  for (int s = 0; s < C::DSTEPS; ++s)
    kro[s] = krow * C::ROWB + (((2 * s + lg) ^ kswz<D>(krow)) * 16);

  // ---- running state: one query per lane (shared by lanes l and l^32) ----
  f32x16 oacc[C::DBLK];
#pragma unroll
  for (int d = 0; d < C::DBLK; ++d) oacc[d] = (f32x16){};
  f32x16 sacc[C::KBLK];   // S(t), from its MFMA phase to its softmax phase
  bf16x8 pf[C::KBLK][2];  // P(t), from its softmax phase to the next MFMA phase
  float m_run = kNegInf;  // running maximum that set the reference (log2 domain)
  float m_use = 0.f;      // exponent reference: m_run, or 0 while m_run = -inf
  float m_thr = kNegInf;  // (m_run + kRescaleSlack) / c_exp: raw score that moves it
  float e_thr = -1.f;     // lane sum of exponentials that calls for the maxima
                          // (kMoveSum; -1, so every tile, while m_run = -inf)
  float l_run = 0.f;      // this lane's part of the running sum
  const float c_exp = p.c_exp;

  // S^T = K Q^T for the tile in K buffer `stage`, fp32 accumulation from 0
  auto qk = [&](int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < C::DSTEPS; ++s)
#pragma unroll
      for (int kb = 0; kb < C::KBLK; ++kb) {
        const bf16x8 a =
            lds_load<bf16x8>(kbuf(stage) + kb * 32 * C::ROWB, kro[s]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            a, qf[s], s == 0 ? (f32x16){} : sacc[kb], 0, 0, 0);
      }
  };
  // O^T += V^T P^T from V buffer `buf`
  auto pv = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int d = 0; d < C::DBLK; ++d) {
          const lds_u8* vb = vbuf(buf) + vtr[d] + (32 * kb + 16 * j) * C::ROWB;
          const bf16x8 va = join_tr16(lds_tr16(vb), lds_tr16(vb + 4 * C::ROWB));
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[kb][j], oacc[d], 0, 0, 0);
        }
  };

  // P(t) = exp2(s*c - m) against the current exponent reference, rounded to bf16 in
  // the B-operand layout of P.V; returns this lane's sum of the exponentials
  auto exps = [&]() __attribute__((always_inline)) {
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4 w;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float e0 =
              __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * j + 2 * x], c_exp, -m_use));
          const float e1 = __builtin_amdgcn_exp2f(
              __builtin_fmaf(sacc[kb][8 * j + 2 * x + 1], c_exp, -m_use));
          lsum += e0 + e1;
          w[x] = pack_bf16x2(e0, e1);
        }
        pf[kb][j] = __builtin_bit_cast(bf16x8, w);
      }
    return lsum;
  };

  // softmax of tile t: mask, exponentials against the current reference, and only when
  // some exponential may exceed 2^kRescaleSlack the row maxima, the lazy correction of
  // O and l and the exponentials again.
  auto softmax = [&](int t, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(mask_tag)::value;
    const int j0 = t * C::BC;
    if (MASKED && (PRE || (j0 + C::BC > L) || (p.causal && j0 + C::BC - 1 > qw))) {
      // key j0 + off of this lane is visible iff off < lim (kv_len and causal bounds)
      const int lim = min(L, p.causal ? qrow + 1 : L) - j0 - 8 * lg;
#pragma unroll
      for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + 16 * (r >> 3) + (r & 7);
          const float x = PRE ? sacc[kb][r] * p.c_pre : sacc[kb][r];
          sacc[kb][r] = off < lim ? x : kNegInf;
        }
    }
    float lsum = exps();
    // A score above the move threshold m_thr has an exponential above e_thr (half of
    // 2^kRescaleSlack, far more than the rounding of the two tests apart), and then so
    // has the lane's sum, every term being >= 0.  So the maxima are needed only when some
    // lane's sum exceeds e_thr; below it no reference of the wave moves, exactly as
    // the test on the maxima would have found.
    if (__builtin_expect(__any(lsum > e_thr), 0)) {
      // guard: a row with no valid key so far keeps m = -inf and uses 0 as its
      // exponent reference, so no -inf - (-inf) is ever formed
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = max_with_partner(mx);
      // compared in the raw score domain
      const bool move = mx > m_thr;
      if (__any(move)) {
        const float m_new = move ? mx * c_exp : m_run;
        const float mu = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = move ? __builtin_amdgcn_exp2f(m_run - mu) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
        m_run = m_new;
        m_use = mu;
        m_thr = (m_run + kRescaleSlack) / c_exp;
        e_thr = m_run == kNegInf ? -1.f : kMoveSum;
        lsum = exps();
      }
    }
    l_run += lsum;
  };

  auto epilogue = [&]() __attribute__((always_inline)) {
  // ---- epilogue: O = a / l (0 for rows with no valid key), LSE = ln2 (m + log2 l) ----
  const float l_tot = sum_with_partner(l_run);
  if (qrow < p.Nq) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    unsigned short* orow = op + (size_t)qrow * D;
#pragma unroll
    for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 w = {pack_bf16x2(oacc[d][4 * a + 0] * inv, oacc[d][4 * a + 1] * inv),
                   pack_bf16x2(oacc[d][4 * a + 2] * inv, oacc[d][4 * a + 3] * inv)};
        *(u32x2*)(orow + d * 32 + 8 * a + 4 * lg) = w;
      }
    if (lg == 0) {
      lsep[qrow] = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : kNegInf;
    }
  }
  };

  // true when no row of this wave sees any key of tile t (wave-uniform)
  auto wave_blind = [&](int t) __attribute__((always_inline)) {
    const int j0 = t * C::BC;
    return j0 >= L || (p.causal && j0 > qw + 31);
  };

  // One tile period of group G; PAR = t & 1 selects the buffers at compile time.
  //   MFMA phase:    G0 requests V(t) into V buffer PAR (last read by G1's P.V(t-2),
  //                  one phase earlier) and K(t+1) into K buffer PAR ^ 1 (last read by
  //                  G1's Q.K^T(t-1), one phase earlier); O += V(t-1) P(t-1) (t > 0),
  //                  S(t) = K(t) Q^T
  //   softmax phase: P(t); G0 waits for V(t) and K(t+1), which both groups read from
  //                  the next phase on
  // The requests go out between the MFMAs of an interior tile, and first otherwise
  // (the products of a boundary tile may be skipped).  G1 moves no data.
  auto period = [&](const int t, auto grp_tag, auto par_tag, auto first_tag, auto mask_tag)
                    __attribute__((always_inline)) {
    constexpr int G = decltype(grp_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    constexpr bool FIRST = decltype(first_tag)::value;
    constexpr bool MASKED = decltype(mask_tag)::value;
    mfma_priority();
    constexpr int NPV = C::KBLK * 2 * C::DBLK, NQK = C::DSTEPS * C::KBLK;
    if (G == 0) {
      load_v(t, PAR);
      load_k(t + 1, PAR ^ 1);
      if (MASKED || FIRST) __builtin_amdgcn_sched_barrier(0);
    }
    if (MASKED) {
      // boundary tiles: a tile none of whose keys this wave's rows see adds exact
      // zeros to O and l, so its products and softmax are skipped (loads and
      // barriers still run: the other waves need the tiles)
      if (!FIRST && !wave_blind(t - 1)) {
        pv(PAR ^ 1);
        schedule_mfma_phase_pv<NPV, 0>();
      }
      if (!wave_blind(t)) {
        qk(PAR);
        schedule_mfma_phase<C::DSTEPS * C::KBLK>();
      }
    } else {
      if (!FIRST) {
        pv(PAR ^ 1);
        qk(PAR);
        schedule_mfma_phase_pv<NPV, NQK, G == 0 ? 2 * C::KDMA : 0>();
      } else {
        qk(PAR);
        schedule_mfma_phase<NQK>();
      }
    }
    phase_barrier();
    valu_priority();
    if (!MASKED || !wave_blind(t)) softmax(t, mask_tag);
    if (G == 0) wait_vm0();   // V(t), K(t+1) have landed: they are read after the barrier
    phase_barrier();
  };

  // The whole key loop of one group, as straight-line code of its own: the two
  // groups move different data, and one shared body would make the compiler merge
  // their register states (and wait for loads the other group issued).
  auto run_group = [&](auto grp_tag) __attribute__((always_inline)) {
    constexpr int G = decltype(grp_tag)::value;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // prologue: K(0) in LDS (V(0) and K(1) are requested in the first period)
    if (n_tiles > 0 && G == 0) load_k(0, 0);
    wait_vm0();   // (and the Q fragments)
    phase_barrier();
    if (n_tiles > 0) {
      if (G == 1) phase_barrier();   // G1 starts one phase late
      using T_ = std::true_type;
      using F_ = std::false_type;
      period(0, grp_tag, I0{}, T_{}, T_{});
      int t = 1;
      // tiles every row of the workgroup sees whole: no mask code at all
      for (; t + 1 < n_full; t += 2) {
        period(t, grp_tag, I1{}, F_{}, F_{});
        period(t + 1, grp_tag, I0{}, F_{}, F_{});
      }
      for (; t + 1 < n_tiles; t += 2) {
        period(t, grp_tag, I1{}, F_{}, T_{});
        period(t + 1, grp_tag, I0{}, F_{}, T_{});
      }
      if (t < n_tiles) period(t, grp_tag, I1{}, F_{}, T_{});
      // last MFMA phase: O += V(n-1) P(n-1)
      mfma_priority();
      if (!wave_blind(n_tiles - 1)) {
        if ((n_tiles - 1) & 1) pv(1);
        else pv(0);
      }
      valu_priority();
      // G0 ends one phase early; it meets G1's last softmax barrier
      if (G == 0) phase_barrier();
    }
    epilogue();
  };

  if (grp == 0) run_group(std::integral_constant<int, 0>{});
  else run_group(std::integral_constant<int, 1>{});
}

}  // namespace

int launch_attn_fwd_bf16_pp(const FwdArgs& a, int D, hipStream_t stream) {
  const int n_qb = (a.Nq + 255) / 256;
  const long long grid = (long long)n_qb * a.B * a.H;
  if (grid > 0x7fffffffLL) return -8;
  const dim3 g((unsigned)grid), blk(512);
  if (D == 128) {
    if (a.pre_scale)
      attn_fwd_bf16_pp_kernel<128, true><<<g, blk, 0, stream>>>(a);
    else
      attn_fwd_bf16_pp_kernel<128, false><<<g, blk, 0, stream>>>(a);
  } else {
    if (a.pre_scale)
      attn_fwd_bf16_pp_kernel<64, true><<<g, blk, 0, stream>>>(a);
    else
      attn_fwd_bf16_pp_kernel<64, false><<<g, blk, 0, stream>>>(a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace attn89
