// attn_fwd_bf16_4w.hip -- the fused attention forward for gfx950, bf16 in / bf16 out,
// 4-wave workgroups, two per CU (head dimension 64, and grids too small for the
// 8-wave ping-pong kernel of attn_fwd_bf16_pp.hip to fill the GPU).
//
// One kernel computes O = softmax(Q K^T * scale + mask) V and the LSE.  The score
// tile, its row maximum and sum, the exponentials, the online correction
// exp(m_old - m_new) and the P.V product never leave the workgroup (page
// "Attention softmax fusion", sections "What fused has to mean" and "The tile
// loop"; page "Kernel Fusion and the Memory Wall", section "FlashAttention: avoid
// the full score matrix").
//
// Work split.  One workgroup = 4 waves = 128 query rows of one (batch, head); each
// wave owns 32 rows for the whole key loop.  Keys are streamed in tiles of 64.  A
// workgroup uses 64 KiB of LDS (D = 128) and at most 256 registers per lane, so two
// workgroups (two waves per SIMD) share a CU and hide each other's latencies.
//
// Register and LDS layouts (transposed scores, P straight from the score registers,
// swizzled K and V tiles) and the lazy online correction are described in
// attn_bf16_tiles.hpp.
//
// Data movement.  K and V tiles go from global memory straight into LDS
// (buffer_load ... lds, no staging registers), row-major, double buffered: the loads
// of tile t+1 are issued before tile t is computed.  The P.V operand (one dimension,
// eight keys per lane) is read from the row-major V tile with transposing
// ds_read_b64_tr_b16 reads, two per fragment (each V buffer is an LDS array of its
// own, so these reads need not wait for the next tile's loads).  The 16-byte chunks of
// each row are
// XOR-swizzled with a function of the row (K and V each their own), so the fragment
// reads are bank-conflict free (the lanes the LDS serves together touch each bank
// once).  The key loop is unrolled by two, so the buffer of every LDS access is known
// at compile time and every fragment address is a per-lane register computed once
// plus an immediate offset: no address arithmetic in the loop.  (V used to pass
// through registers and be written transposed with byte permutes: 16 vector
// instructions per tile and thread, which the D = 64 tiles, bound by vector work,
// paid for: the transposing reads gained 5-9 % there, same bits.)
//
// Key tile t:
//   a) issue the loads of K(t+1) and V(t+1) (LDS)
//   b) S(t) = K(t) Q^T on the matrix cores
//   c) mask S(t) if the tile reaches past kv_len or crosses the causal diagonal
//   d) row maxima -> exponent reference m(t); if a reference moved, O and l are
//      multiplied by alpha(t) (rare, see attn_bf16_tiles.hpp)
//   e) P(t) = exp2(S(t)*c - m(t)), its row sums and its bf16 packing
//   f) O^T += V(t)^T P(t)^T on the matrix cores
//   g) barrier (K(t+1) and V(t+1) have landed)
// The two workgroups on a CU interleave these phases, so one wave's exponentials
// run while the other's matrix instructions do.
//
#include <type_traits>

#include "attn_bf16_tiles.hpp"
#include "launch.hpp"
#include "mfma_schedule.hpp"

namespace attn89 {
namespace {

template <int D, int RW = 4>
struct Cfg {
  static constexpr int BR = 32 * RW;             // query rows per workgroup (RW waves of 32)
  static constexpr int BC = 64;                  // keys per tile
  static constexpr int NT = 64 * RW;             // threads per key group
  static constexpr int ROWB = D * 2;             // bytes per K row
  static constexpr int TILE = BC * ROWB;         // bytes per K (or V) tile
  static constexpr int DMA = TILE / 1024 / RW;   // 1 KiB K loads per wave per tile
  static constexpr int DSTEPS = D / 16;          // k-steps of S^T = K Q^T
  static constexpr int DBLK = D / 32;            // 32-dimension blocks of O^T
  static constexpr int KBLK = BC / 32;           // 32-key blocks of a tile
  static constexpr int OX = DBLK * 16 * NT * 4;  // bytes of one key group's O (fp32)
  static_assert((BC / 4) * (D / 8) <= NT || NT == 256, "V staging: one unit a thread");
};

// PRE: scale <= 0, so scores are scaled before they are masked (a separate
// instantiation keeps that branch out of the common kernel).
// SPLIT: the workgroup covers one key range of the row block and writes a partial
// result (normalised O_r in fp32 and LSE_r) for the merge of attn_splitkv.hip.
// VARLEN: packed variable-length sequences (FwdArgs cu_q, cu_k): Q, K, V and O are
// [tokens][H][D], sequence b owns tokens [cu[b], cu[b+1]), rows are H*D apart; Nq
// and Nk are the longest sequence lengths the grid and the checks were sized for.
// KS, RW: key groups per workgroup and row waves per group.  The plain kernel is
// KS = 1, RW = 4 (four waves, 128 rows).  With KS > 1 the workgroup has KS groups of
// RW waves; every group covers the same 32*RW query rows, group g takes the key tiles
// t = g, g + KS, ... (each group with its own K / V double buffers), and at the end
// groups 1 .. KS-1 hand their (O, m, l) to group 0 through LDS, where they are combined
// with the same rescaling as any reference move.  For grids too small to fill the GPU:
// KS = 2, RW = 4 halves the sequential key loop of a 128-row block (D = 128); KS = 2,
// RW = 2 (D = 64) also halves the rows of a block, so two workgroups share a CU and the
// heavy causal blocks spread over twice as many CUs.
template <int D, bool PRE, bool SPLIT, bool VARLEN, int KS, int RW>
__global__ __launch_bounds__(64 * RW * KS, KS == 1 ? 2 : (64 * RW * KS >= 512 ? 1 : 2))
void attn_fwd_bf16_4w_kernel(FwdArgs p) {
  static_assert(!(SPLIT && VARLEN), "split keys over packed sequences is not provided");
  static_assert(KS == 1 || (!SPLIT && !VARLEN), "key groups only in the plain kernel");
  static_assert(RW == 4 || KS > 1, "fewer row waves only with key groups");
  static_assert(KS * RW <= 8, "at most 8 waves a workgroup");
  using C = Cfg<D, RW>;
  // Each of the four tile buffers (K and V, double buffered; one slot per key group)
  // is an LDS array of its own: a fragment read of one buffer while a DMA into the
  // other is in flight must not look like a possible overlap to the compiler, which
  // would wait for the outstanding loads first (see attn_bf16_tiles.hpp).
  __shared__ __attribute__((aligned(1024))) unsigned char smem_k0[C::TILE * KS];
  __shared__ __attribute__((aligned(1024))) unsigned char smem_k1[C::TILE * KS];
  __shared__ __attribute__((aligned(1024))) unsigned char smem_v0[C::TILE * KS];
  __shared__ __attribute__((aligned(1024))) unsigned char smem_v1[C::TILE * KS];
  static_assert(KS <= 2, "the O exchange below is written for two key groups");
  static_assert(KS == 1 || C::OX / 2 <= C::TILE * KS, "half of a key group's O fits a K buffer");
  static_assert(KS == 1 || 3 * C::NT * 4 <= C::TILE * KS, "row statistics fit a V buffer");
  const int tid = threadIdx.x;
  // wave-uniform values in scalar registers (branches on them must be real branches:
  // every wave meets every barrier)
  const int wave = KS == 1 ? (tid >> 6) : (__builtin_amdgcn_readfirstlane(tid >> 6) % RW);
  const int kgrp = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6) / RW;   // key group
  const int tid_g = tid % C::NT;                   // thread inside its key group
  // buffer `buf` of a tile array; this key group's slot starts goff bytes in (added to
  // the DMA targets and folded into the per-lane fragment offsets)
  auto kbuf = [&](int buf) __attribute__((always_inline)) {
    return buf ? (lds_u8*)smem_k1 : (lds_u8*)smem_k0;
  };
  auto vbuf = [&](int buf) __attribute__((always_inline)) {
    return buf ? (lds_u8*)smem_v1 : (lds_u8*)smem_v0;
  };
  const unsigned goff = (unsigned)kgrp * C::TILE;
  const int lane = tid & 63;
  const int lq = lane & 31;   // query column inside the wave's 32 rows
  const int lg = lane >> 5;   // half of the wave

  // Schedule.  Workgroups are dispatched to the 8 XCDs round robin, so when B*H is a
  // multiple of 8 every query block of a head lands on one XCD and its K/V re-reads
  // can stay in that XCD's L2.  Causal (or split-key) calls: consecutive workgroups
  // take different (b, h) of the same query block, heaviest (last) blocks first,
  // which balances blocks of unequal length.  Otherwise every block of a head has the
  // same length and each XCD takes its heads one at a time, all query blocks of one
  // head before the next, so few heads' K/V compete for its L2.
  const int BH = p.B * p.H;
  const int n_qb = (p.Nq + C::BR - 1) / C::BR;
  const int split = SPLIT ? (int)blockIdx.x % p.n_splits : 0;
  const int wg_id = SPLIT ? (int)blockIdx.x / p.n_splits : (int)blockIdx.x;
  int qb, bh;
  if (!SPLIT && !p.causal && BH % 8 == 0) {
    const int x = wg_id % 8, slot = wg_id / 8;
    bh = x + 8 * (slot / n_qb);
    qb = n_qb - 1 - slot % n_qb;
  } else if (KS > 1 && KS * RW * 64 * 2 <= 512) {
    // two workgroups per CU, all resident at once (the dispatcher places workgroups
    // t and t + grid/2 on the same CU): the first half of the grid takes the causal
    // blocks longest first, the second half shortest first, so the two workgroups of a
    // CU add up to about the same work on every CU
    const int s = wg_id / BH, half = (n_qb + 1) / 2;
    bh = wg_id % BH;
    qb = s < half ? n_qb - 1 - s : s - half;
  } else {
    qb = n_qb - 1 - wg_id / BH;
    bh = wg_id % BH;
  }
  const int b = bh / p.H;

  // rows of this (batch, head): nq queries and L valid keys, ld elements apart
  const int ld = VARLEN ? p.H * D : D;
  size_t qbase, kbase;
  int nq, L;
  float* lsep;
  if (VARLEN) {
    const int h = bh % p.H;
    const SeqSpan sq = seq_span(p.cu_q, b, p.total_q, p.Nq);
    const SeqSpan sk = seq_span(p.cu_k, b, p.total_k, p.Nk);
    nq = sq.len;
    L = sk.len;
    qbase = (size_t)sq.start * ld + (size_t)h * D;
    kbase = (size_t)sk.start * ld + (size_t)h * D;
    lsep = p.lse + (size_t)h * p.total_q + sq.start;
    if (qb * C::BR >= nq) return;   // the whole workgroup: past this sequence's queries
  } else {
    nq = p.Nq;
    L = clamp_len(p.kv_lens, b, p.Nk);              // valid keys of this sequence
    qbase = (size_t)bh * p.Nq * D;
    kbase = (size_t)bh * p.Nk * D;
    lsep = p.lse + (size_t)bh * p.Nq;
  }
  const unsigned short* qp = (const unsigned short*)p.q + qbase;
  const unsigned short* kp = (const unsigned short*)p.k + kbase;
  const unsigned short* vp = (const unsigned short*)p.v + kbase;
  unsigned short* op = (unsigned short*)p.o + qbase;

  const int q0 = qb * C::BR;
  const int q_hi = min(q0 + C::BR, nq);
  const int kv_end = p.causal ? min(L, q_hi) : L;    // keys any row of the block sees
  const int n_tiles_all = (kv_end + C::BC - 1) / C::BC;
  // key tiles [t_begin, n_tiles) of this workgroup (all of them unless split)
  const int t_begin = SPLIT ? split * (p.kv_chunk / C::BC) : 0;
  const int n_tiles = SPLIT ? min(n_tiles_all, t_begin + p.kv_chunk / C::BC) : n_tiles_all;
  // leading tiles whose keys are all visible to every row of the block
  const int n_full = PRE ? 0 : min(L, p.causal ? q0 + 1 : L) / C::BC;
  const int qw = q0 + wave * 32;                     // first row of this wave
  const int qrow = qw + lq;

  // ---- Q fragments (B operand of S^T = K Q^T), resident for the whole loop ----
  // Buffer loads: rows past Nq (and below, keys past kv_len) read as zeros.
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qp, (unsigned)((nq - 1) * ld + D) * 2);
  bf16x8 qf[C::DSTEPS];
#pragma unroll
  for (int s = 0; s < C::DSTEPS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8,
                               buffer_load16(qrs, ((unsigned)qrow * ld + 16 * s + 8 * lg) * 2));

  // ---- K: global -> LDS without registers ----
  // Load n of this wave writes tile bytes [m*1024, m*1024 + 1024), m = wave*DMA + n,
  // lane i the 16 bytes at m*1024 + 16*i; the lane fetches the global chunk the
  // swizzle puts there.  The tile start is the scalar offset of the load.
  // rows past L read as zeros (the last valid row ends at (L - 1) * ld + D)
  const unsigned kv_bytes = L > 0 ? (unsigned)((L - 1) * ld + D) * 2 : 0u;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, kv_bytes);
  unsigned koff[C::DMA];
#pragma unroll
  for (int n = 0; n < C::DMA; ++n) {
    const int byte = (wave * C::DMA + n) * 1024 + 16 * lane;
    const int row = byte / C::ROWB;
    const int ch = ((byte % C::ROWB) / 16) ^ kswz<D>(row);
    koff[n] = ((unsigned)row * ld + 8 * ch) * 2;
  }
  auto load_k = [&](int t, int stage) {
#pragma unroll
    for (int n = 0; n < C::DMA; ++n)
      buffer_load16_to_lds(krs, (lds_void*)(kbuf(stage) + goff + (wave * C::DMA + n) * 1024),
                           koff[n], t * C::BC * ld * 2);
  };

  // ---- V: global -> LDS without registers, row-major ----
  // The P.V operand (one dimension per lane, the 8 keys of its P fragment) is read back
  // with the transposing ds_read_b64_tr_b16 (see lds_tr16): the lane at position
  // i = 4m + a of a group of 16 lanes (group g) addresses, in read q, key
  // 8(g/2) + 4q + m (plus the P.V step's 16-key offset) at dimensions
  // 16(g%2) + 4a .. + 4 of the 32-dimension block, so two reads give a lane its 8
  // elements.  V rows keep their 16-byte chunks XOR-swizzled by vswz(row), which
  // depends on row bits 0-1 only: the four keys one read gathers then fall in different
  // 64-byte windows (no bank conflicts), and key offsets of 4, 16 and 32 keep the
  // swizzle, so they are immediate offsets.
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, kv_bytes);
  unsigned voff[C::DMA];
#pragma unroll
  for (int n = 0; n < C::DMA; ++n) {
    const int byte = (wave * C::DMA + n) * 1024 + 16 * lane;
    const int row = byte / C::ROWB;
    const int ch = ((byte % C::ROWB) / 16) ^ vswz<D>(row);
    voff[n] = ((unsigned)row * ld + 8 * ch) * 2;
  }
  auto load_v = [&](int t, int stage) {
#pragma unroll
    for (int n = 0; n < C::DMA; ++n)
      buffer_load16_to_lds(vrs,
                           (lds_void*)(vbuf(stage) + goff + (wave * C::DMA + n) * 1024),
                           voff[n], t * C::BC * ld * 2);
  };
  unsigned vtr[C::DBLK];   // read q of 32-dimension block d at P.V step s: + (16 s + 4 q) rows
  {
    const int gi = lane & 15, gg = lane >> 4, a = gi & 3, m = gi >> 2;
    const int key = 8 * (gg >> 1) + m;
#pragma unroll
    for (int d = 0; d < C::DBLK; ++d)
      vtr[d] = goff + key * C::ROWB + (((4 * d + 2 * (gg & 1) + (a >> 1)) ^ vswz<D>(key)) * 16) +
               8 * (a & 1);
  }

  // ---- fragment read offsets (per lane, fixed for the whole loop) ----
  const int krow = swap_bits23(lq);   // key (row of K) this lane feeds to the MFMA
  unsigned kro[C::DSTEPS];
#pragma unroll
  for (int s = 0; s < C::DSTEPS; ++s)
    kro[s] = goff + krow * C::ROWB + (((2 * s + lg) ^ kswz<D>(krow)) * 16);

  // S^T = K Q^T for the tile in K buffer `stage`, fp32 accumulation from 0
  auto qk = [&](int stage, f32x16* sacc) {
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

  // mask of tile t: -inf for keys past kv_len and keys above the causal diagonal
  auto needs_mask = [&](int t) {
    const int j0 = t * C::BC;
    return PRE || (j0 + C::BC > L) || (p.causal && j0 + C::BC - 1 > qw);
  };
  auto apply_mask = [&](int t, f32x16* sacc) {
    // key j0 + off of this lane is visible iff off < lim (kv_len and causal bounds)
    const int lim = min(L, p.causal ? qrow + 1 : L) - t * C::BC - 8 * lg;
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = kb * 32 + 16 * (r >> 3) + (r & 7);
        const float x = PRE ? sacc[kb][r] * p.c_pre : sacc[kb][r];
        sacc[kb][r] = off < lim ? x : kNegInf;
      }
  };

  // ---- running state: one query per lane (shared by lanes l and l^32) ----
  f32x16 oacc[C::DBLK];
#pragma unroll
  for (int d = 0; d < C::DBLK; ++d) oacc[d] = (f32x16){};
  float m_run = kNegInf;  // running maximum that set the reference (log2 domain)
  float m_use = 0.f;      // exponent reference: m_run, or 0 while m_run = -inf
  float m_thr = kNegInf;  // (m_run + kRescaleSlack) / c_exp: raw score that moves it
  float e_thr = -1.f;     // lane sum of exponentials that calls for the maxima
                          // (kMoveSum; -1, so every tile, while m_run = -inf)
  float l_run = 0.f;      // this lane's part of the running sum
  const float c_exp = p.c_exp;

  // ---- one key tile; PAR = t & 1 selects the buffers at compile time ----
  auto iteration = [&](const int t, auto par_tag, auto last_tag, auto mask_tag,
                       const int tstep = 1) {
    constexpr bool MASKED = decltype(mask_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    constexpr bool LAST = decltype(last_tag)::value;
    // a) prefetch the next tile of this workgroup (key group)
    if (!LAST) {
      load_k(t + tstep, PAR ^ 1);
      load_v(t + tstep, PAR ^ 1);
    }
    // b) scores; c) mask
    f32x16 scur[C::KBLK];
    qk(PAR, scur);
    schedule_mfma_run<C::DSTEPS * C::KBLK, 1, LAST ? 0 : 2 * C::DMA, 4>();
    if (MASKED && needs_mask(t)) apply_mask(t, scur);
    // d) P = exp2(s*c - m) against the current exponent reference, rounded to bf16 in
    //    the B-operand layout of O^T = V^T P^T; lsum = this lane's sum of the exponentials
    bf16x8 pf[C::KBLK][2];
    auto exps = [&]() {
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          u32x4 w;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const float e0 = __builtin_amdgcn_exp2f(
                __builtin_fmaf(scur[kb][8 * j + 2 * x], c_exp, -m_use));
            const float e1 = __builtin_amdgcn_exp2f(
                __builtin_fmaf(scur[kb][8 * j + 2 * x + 1], c_exp, -m_use));
            lsum += e0 + e1;
            w[x] = pack_bf16x2(e0, e1);
          }
          pf[kb][j] = __builtin_bit_cast(bf16x8, w);
        }
      return lsum;
    };
    float lsum = exps();
    // e) a score above the move threshold m_thr has an exponential above e_thr, and so
    //    has its lane's sum (every term >= 0): only when some lane's sum exceeds e_thr
    //    are the row maxima (in-lane, then with the partner lane) formed and the
    //    reference tested; below it none would move.  Guard: a row with no valid key
    //    so far keeps m = -inf and uses 0 as its exponent reference, so no
    //    -inf - (-inf) is ever formed.
    if (__builtin_expect(__any(lsum > e_thr), 0)) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, scur[kb][r]);
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
    // f) O^T += V^T P^T from V buffer PAR (P.V step 2kb + j covers keys 32kb + 16j ..)
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int d = 0; d < C::DBLK; ++d) {
          const lds_u8* vb = vbuf(PAR) + vtr[d] + (32 * kb + 16 * j) * C::ROWB;
          const bf16x8 va = join_tr16(lds_tr16(vb), lds_tr16(vb + 4 * C::ROWB));
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[kb][j], oacc[d], 0, 0, 0);
        }
    schedule_mfma_run<C::KBLK * 2 * C::DBLK, 2, 0, 4>();
    // g) the next tile must be in LDS before any wave goes on (with key groups the
    //    caller holds the barrier, met by every group)
    if (!LAST && KS == 1) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's K(t+1), V(t+1) landed
      __syncthreads();
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  if constexpr (KS == 1) {
    // ---- prologue: K(t_begin) and V(t_begin) in LDS ----
    if (n_tiles > t_begin) {
      load_v(t_begin, 0);
      load_k(t_begin, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): also drains the Q fragments
    __syncthreads();
    int t = t_begin;
    // tiles every row of the workgroup sees whole: no mask code at all
    for (; t + 2 < n_tiles && t + 1 < n_full; t += 2) {
      iteration(t, I0{}, F_{}, F_{});
      iteration(t + 1, I1{}, F_{}, F_{});
    }
    for (; t + 2 < n_tiles; t += 2) {
      iteration(t, I0{}, F_{}, T_{});
      iteration(t + 1, I1{}, F_{}, T_{});
    }
    if (t + 1 < n_tiles) {
      iteration(t, I0{}, F_{}, T_{});
      iteration(t + 1, I1{}, T_{}, T_{});
    } else if (t < n_tiles) {
      iteration(t, I0{}, T_{}, T_{});
    }
  } else {
    // group kgrp: tiles my_first, my_first + KS, ...; every group runs n_steps steps
    // (a group past its last tile only meets the barriers)
    const int my_first = t_begin + kgrp;
    const int n_steps = (n_tiles - t_begin + KS - 1) / KS;
    if (my_first < n_tiles) {
      load_v(my_first, 0);
      load_k(my_first, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    auto step = [&](int i, auto par_tag) {
      const int t = my_first + KS * i;
      const bool more = i + 1 < n_steps;            // uniform over the workgroup
      if (t < n_tiles) {
        if (t + KS < n_tiles) iteration(t, par_tag, F_{}, T_{}, KS);
        else iteration(t, par_tag, T_{}, T_{}, KS);
      }
      if (more) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        __syncthreads();
      }
    };
    for (int i = 0; i < n_steps; i += 2) {
      step(i, I0{});
      if (i + 1 < n_steps) step(i + 1, I1{});
    }
    // hand the (O, m, l) of group 1 to group 0: the K buffers take its O (the first
    // half of the 32-dimension blocks in one, the rest in the other), the first V
    // buffers the row statistics (all buffers are free once every group has left the
    // loop)
    __syncthreads();
    float* s_x = (float*)smem_v0;
    auto o_x = [&](int d) __attribute__((always_inline)) {
      constexpr int HB = C::DBLK / 2;
      return (float*)(d < HB ? (lds_u8*)smem_k0 : (lds_u8*)smem_k1) + (d % HB) * 16 * C::NT;
    };
    const int slot = wave * 64 + lane;             // < 64 * RW
    if (kgrp > 0) {
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o_x(d)[r * C::NT + slot] = oacc[d][r];
      float* st = s_x + (kgrp - 1) * 3 * C::NT;
      st[slot] = m_run;
      st[C::NT + slot] = m_use;
      st[2 * C::NT + slot] = l_run;
    }
    __syncthreads();
    if (kgrp > 0) return;                           // no barrier follows
    float M = m_run;
#pragma unroll
    for (int g = 1; g < KS; ++g) M = fmaxf(M, s_x[(g - 1) * 3 * C::NT + slot]);
    if (M != kNegInf) {
      // every part is rescaled to the largest reference (a part without any valid key
      // has weight 0), the same correction as a reference move
      const float f0 = m_run == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_use - M);
      l_run *= f0;
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= f0;
#pragma unroll
      for (int g = 1; g < KS; ++g) {
        const float* st = s_x + (g - 1) * 3 * C::NT;
        const float mg = st[slot], mug = st[C::NT + slot], lg_ = st[2 * C::NT + slot];
        const float fg = mg == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mug - M);
        l_run += lg_ * fg;
#pragma unroll
        for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[d][r] += o_x(d)[r * C::NT + slot] * fg;
      }
      m_run = M;
      m_use = M;
    }
  }

  // ---- epilogue: O = a / l (0 for rows with no valid key), LSE = ln2 (m + log2 l) ----
  const float l_tot = sum_with_partner(l_run);
  if (SPLIT) {
    // partial result of this key range, fp32 for the merge (an empty range gives
    // O_r = 0 and LSE_r = -inf, weight 0 in the merge)
    if (qrow < nq) {
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      const size_t row = ((size_t)split * BH + bh) * p.Nq + qrow;
      float* orow = p.o_part + row * D;
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *(f32x4*)(orow + d * 32 + 8 * a + 4 * lg) =
              (f32x4){oacc[d][4 * a + 0] * inv, oacc[d][4 * a + 1] * inv,
                      oacc[d][4 * a + 2] * inv, oacc[d][4 * a + 3] * inv};
      if (lg == 0)
        p.lse_part[row] = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : kNegInf;
    }
    return;
  }
  if (qrow < nq) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    unsigned short* orow = op + (size_t)qrow * ld;
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
}

}  // namespace

template <bool SPLIT, bool VARLEN, int KS, int RW>
static int launch_4w(const FwdArgs& a, int D, hipStream_t stream) {
  const int n_qb = (a.Nq + 32 * RW - 1) / (32 * RW);
  const long long grid = (long long)n_qb * a.B * a.H * (SPLIT ? a.n_splits : 1);
  if (grid > 0x7fffffffLL) return -8;
  const dim3 g((unsigned)grid), blk(64 * RW * KS);
  if (D == 128) {
    if constexpr (RW == 4) {
      if (a.pre_scale)
        attn_fwd_bf16_4w_kernel<128, true, SPLIT, VARLEN, KS, RW><<<g, blk, 0, stream>>>(a);
      else
        attn_fwd_bf16_4w_kernel<128, false, SPLIT, VARLEN, KS, RW><<<g, blk, 0, stream>>>(a);
    } else {
      return -3;   // D = 128 key groups use four row waves
    }
  } else {
    if (a.pre_scale)
      attn_fwd_bf16_4w_kernel<64, true, SPLIT, VARLEN, KS, RW><<<g, blk, 0, stream>>>(a);
    else
      attn_fwd_bf16_4w_kernel<64, false, SPLIT, VARLEN, KS, RW><<<g, blk, 0, stream>>>(a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int launch_attn_fwd_bf16_4w(const FwdArgs& a, int D, hipStream_t stream, int key_groups) {
  if (key_groups == 2) {
    // D = 64: 64-row blocks, two key groups of two row waves (4 waves, two workgroups
    // per CU); D = 128: 128-row blocks, two key groups of four row waves (each group's
    // K / V buffers take 64 KiB of LDS, one workgroup per CU)
    if (D == 64) return launch_4w<false, false, 2, 2>(a, D, stream);
    return launch_4w<false, false, 2, 4>(a, D, stream);
  }
  return launch_4w<false, false, 1, 4>(a, D, stream);
}

int launch_attn_fwd_bf16_4w_split(const FwdArgs& a, int D, hipStream_t stream) {
  return launch_4w<true, false, 1, 4>(a, D, stream);
}

int launch_attn_fwd_bf16_4w_varlen(const FwdArgs& a, int D, hipStream_t stream) {
  return launch_4w<false, true, 1, 4>(a, D, stream);
}

}  // namespace attn89
