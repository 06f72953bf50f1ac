// attn_fwd_bf16.hip -- the fused attention forward for gfx950, bf16 in / bf16 out.
//
// One kernel computes O = softmax(Q K^T * scale + mask) V and the LSE.  The score
// tile, its row maximum and sum, the exponentials, the online correction
// exp(m_old - m_new) and the P.V product never leave the workgroup (page
// "Attention softmax fusion", sections "What fused has to mean" and "The tile
// loop"; page "Kernel Fusion and the Memory Wall", section "FlashAttention: avoid
// the full score matrix").
//
// Work split: one workgroup = 4 waves = BR = 128 query rows of one (batch, head);
// each wave owns 32 rows for the whole key loop.  Keys are streamed in tiles of
// BC = 64 through LDS, double buffered: the global loads of tile t+1 are issued
// before tile t is computed and written to the other LDS buffer after it.
//
// Register layout (the core of the design).  A wave computes the TRANSPOSED score
// tile S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the A operand is K (rows = keys,
// from LDS), the B operand is Q^T (columns = queries, held in VGPRs for the whole
// loop).  In the 32x32 accumulator, lane l holds query column l%32 and 16 key rows,
// so each query's scores live in two lanes (l and l^32): the row maximum is an
// in-lane max plus one exchange with lane l^32, the row sum stays per lane until the
// epilogue, and the per-query rescale of the output is a per-lane scalar.
//
// The output is accumulated transposed as well, O^T = V^T P^T, so P is consumed
// straight from the score accumulator registers as the B operand: register 8j+t of
// lane l supplies contraction slot (l/32, t) of the j-th 16-key step.  For that the
// contraction slot of the A operand (V^T, read from LDS) must name the same key,
// and the score rows are therefore produced in a permuted key order: accumulator
// row i is key swap_bits23(i) (bits 2 and 3 of the row index exchanged).  With that
// permutation register r of lane l holds key 16*(r/8) + 8*(l/32) + r%8 of its
// 32-key block, so the 8 keys each lane contributes to a P.V step are consecutive
// and the matching V^T operand is one 16-byte LDS read.  V is transposed once, on
// its way into LDS ([D][BC] layout), so no transpose happens in the inner loop.
//
// LDS rows are padded by 16 bytes so the 16-byte fragment reads of 16 lanes cover
// all 64 banks without conflict.

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace attn89 {
namespace {

template <int D>
struct Cfg {
  static constexpr int BR = 128;           // query rows per workgroup
  static constexpr int BC = 64;            // keys per tile
  static constexpr int NT = 256;           // threads per workgroup (4 waves)
  static constexpr int KSTR = D + 8;       // K tile row stride (bf16 elements)
  static constexpr int VSTR = BC + 8;      // V^T tile row stride (bf16 elements)
  static constexpr int K_ELEMS = BC * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int K_UNITS = BC * D / 8;          // 16-byte units of a K tile
  static constexpr int K_PER_T = K_UNITS / NT;
  static constexpr int V_UNITS = (BC / 4) * (D / 8);  // units of 4 keys x 8 dims
  static constexpr int V_PER_T = (V_UNITS + NT - 1) / NT;
  static constexpr int DSTEPS = D / 16;    // k-steps of the S^T product
  static constexpr int DBLK = D / 32;      // 32-row blocks of O^T
  static constexpr int KBLK = BC / 32;     // 32-key blocks of a tile
};

// v_permlane32_swap exchanges the upper half-wave of one operand with the lower
// half-wave of the other; with both operands = x, the two results of every lane are
// x[l] and x[l ^ 32] (in some order), so their max / sum is the two-lane reduction.
__device__ __forceinline__ float max_with_partner(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_with_partner(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

#ifndef ATTN89_RESCALE_SLACK
#define ATTN89_RESCALE_SLACK 0.0f
#endif
// How far (log2 units) the row maximum may rise above the exponent reference
// before the accumulators are corrected; 0 corrects on every rise.
constexpr float kRescaleSlack = ATTN89_RESCALE_SLACK;

__device__ __forceinline__ int swap_bits23(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(FwdArgs p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) unsigned short smem[2 * (C::K_ELEMS + C::V_ELEMS)];
  // buffer x: K tile at smem + x*K_ELEMS, V^T tile at smem + 2*K_ELEMS + x*V_ELEMS

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;   // query column inside the wave's 32 rows
  const int lg = lane >> 5;   // half of the wave

  // Schedule: consecutive workgroups take different (b, h) of the same query block,
  // heaviest (last, for causal) query blocks first.  Workgroups are dispatched to
  // the 8 XCDs round robin, so when B*H is a multiple of 8 every query block of a
  // head lands on the same XCD and its K/V re-reads stay in that XCD's L2.
  const int BH = p.B * p.H;
  const int n_qb = (p.Nq + C::BR - 1) / C::BR;
  const int t_id = blockIdx.x;
  const int qb = n_qb - 1 - t_id / BH;
  const int bh = t_id % BH;
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
  const int qw = q0 + wave * 32;

  // ---- Q fragments: B operand of S^T = K Q^T, resident for the whole loop ----
  // Buffer loads: rows past Nq (or keys past kv_len below) read as zeros.
  const int qrow = qw + lq;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qp, (unsigned)p.Nq * D * 2);
  bf16x8 qf[C::DSTEPS];
#pragma unroll
  for (int s = 0; s < C::DSTEPS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8, buffer_load16(qrs, ((unsigned)qrow * D + 16 * s + 8 * lg) * 2));

  // ---- tile staging: global -> registers -> LDS ----
  // K runs one tile ahead of V: while tile t is exponentiated and multiplied into O,
  // the scores of tile t+1 are already being produced.  Iteration t reads K(t+1)
  // from K buffer (t+1)&1 and V(t) from V buffer t&1, and writes K(t+2) into K
  // buffer t&1 and V(t+1) into V buffer (t+1)&1; one barrier per iteration.
  u32x4 kreg[C::K_PER_T];
  u32x4 vreg[C::V_PER_T][4];

  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (unsigned)L * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, (unsigned)L * D * 2);
  auto load_k = [&](int j0) {
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int c = tid + C::NT * i;
      const int row = c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      kreg[i] = buffer_load16(krs, ((unsigned)(j0 + row) * D + col) * 2);
    }
  };
  auto load_v = [&](int j0) {
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int u = tid + C::NT * i;
      const int kg = u % (C::BC / 4);
      const int dg = u / (C::BC / 4);
      if (u < C::V_UNITS) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vreg[i][r] = buffer_load16(vrs, ((unsigned)(j0 + 4 * kg + r) * D + 8 * dg) * 2);
      }
    }
  };
  auto store_k = [&](int buf) {
    unsigned short* ks = smem + buf * C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int c = tid + C::NT * i;
      const int row = c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      *(u32x4*)(ks + row * C::KSTR + col) = kreg[i];
    }
  };
  auto store_v = [&](int buf) {
    unsigned short* vt = smem + 2 * C::K_ELEMS + buf * C::V_ELEMS;
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int u = tid + C::NT * i;
      if (u < C::V_UNITS) {
        const int kg = u % (C::BC / 4);
        const int dg = u / (C::BC / 4);
        // 4 keys x 8 dims in registers -> 8 rows of V^T, 4 consecutive keys each
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          const int sh = (e & 1) * 16;
          const unsigned int a0 = (vreg[i][0][w] >> sh) & 0xFFFFu;
          const unsigned int a1 = (vreg[i][1][w] >> sh) & 0xFFFFu;
          const unsigned int a2 = (vreg[i][2][w] >> sh) & 0xFFFFu;
          const unsigned int a3 = (vreg[i][3][w] >> sh) & 0xFFFFu;
          u32x2 pk = {a0 | (a1 << 16), a2 | (a3 << 16)};
          *(u32x2*)(vt + (8 * dg + e) * C::VSTR + 4 * kg) = pk;
        }
      }
    }
  };

  const int krow_perm = swap_bits23(lq);
  // S^T = K Q^T for the 64 keys held in K buffer kbuf, fp32 accumulation
  auto qk = [&](int kbuf, f32x16* sacc) {
    const unsigned short* kbase = smem + kbuf * C::K_ELEMS + krow_perm * C::KSTR + 8 * lg;
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb) sacc[kb] = (f32x16){};
    // consecutive matrix instructions go to different accumulators
#pragma unroll
    for (int s = 0; s < C::DSTEPS; ++s)
#pragma unroll
      for (int kb = 0; kb < C::KBLK; ++kb) {
        const bf16x8 a = *(const bf16x8*)(kbase + kb * 32 * C::KSTR + 16 * s);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
      }
  };

  // ---- running state: one query per lane (shared by lanes l and l^32) ----
  f32x16 oacc[C::DBLK];
#pragma unroll
  for (int d = 0; d < C::DBLK; ++d) oacc[d] = (f32x16){};
  float m_run = kNegInf;  // exponent reference: running max of s*c (log2 domain)
  float l_run = 0.f;      // this lane's part of the running sum
  const float c_exp = p.c_exp;

  f32x16 scur[C::KBLK];   // raw scores of the tile being finished
  if (n_tiles > 0) {
    load_k(0);
    load_v(0);
    store_k(0);
    store_v(0);
    if (n_tiles > 1) {
      load_k(C::BC);
      store_k(1);
    }
  }
  // Drain every outstanding global load (the Q fragments included) before the loop,
  // so inside it the only loads in flight are prefetches and no matrix instruction
  // waits on them.  Encoding: vmcnt(0), expcnt and lgkmcnt unconstrained.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if (n_tiles > 0) qk(0, scur);
  __syncthreads();  // K buffer 0 is rewritten in iteration 0

  // One iteration of the key loop.  LAST (the final tile) has no next tile to
  // score; keeping it a compile-time case leaves the steady-state body free of
  // branches around the matrix work.
  auto iteration = [&](const int t, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    const int j0 = t * C::BC;
    if (!LAST) {
      if (t + 2 < n_tiles) load_k(j0 + 2 * C::BC);
      load_v(j0 + C::BC);
    }

    if (p.pre_scale) {
#pragma unroll
      for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) scur[kb][r] *= p.c_pre;
    }
    // mask: only tiles that reach past kv_len or cross the wave's causal diagonal
    if ((j0 + C::BC > L) || (p.causal && j0 + C::BC - 1 > qw)) {
#pragma unroll
      for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + kb * 32 + 16 * (r >> 3) + 8 * lg + (r & 7);
          const bool ok = key < L && (!p.causal || key <= qrow);
          if (!ok) scur[kb][r] = kNegInf;
        }
    }

    // row maximum: in-lane, then with the partner lane holding the other 16 keys
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, scur[kb][r]);
    mx = max_with_partner(mx) * c_exp;
    // Online correction.  The exponent reference m_run moves to the new maximum when
    // the maximum rises by more than kRescaleSlack (log2 units; 0 = on every rise).
    // Numerator and normaliser always share one reference, so a / l is unchanged;
    // moving the reference multiplies both by alpha = exp2(m_old - m_new), exactly
    // the correction of the recurrence.
    const bool move = mx > m_run + kRescaleSlack;
    const float m_new = move ? mx : m_run;
    // guard: a row with no valid key so far keeps m_new = -inf; use 0 as the
    // exponent reference so that no -inf - (-inf) appears
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;

    if (__any(move)) {
      // alpha == 1 exactly on rows whose reference did not move
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
    }

    // scores of the next tile: independent matrix work that overlaps the
    // exponentials below (same basic block, so the scheduler can interleave them)
    f32x16 snext[C::KBLK];
    if (!LAST) qk((t + 1) & 1, snext);

    // P = exp2(s*c - m), rounded to bf16 as the B operand of O^T = V^T P^T, and the
    // row-sum part of this lane
    bf16x8 pf[C::KBLK][2];
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
    l_run += lsum;

    // O^T += V^T P^T from V buffer t&1; consecutive matrix instructions go to
    // different accumulators and share their B operand
    const unsigned short* vbase = smem + 2 * C::K_ELEMS + (t & 1) * C::V_ELEMS +
                                  lq * C::VSTR + 8 * lg;
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int d = 0; d < C::DBLK; ++d) {
          const bf16x8 a = *(const bf16x8*)(vbase + d * 32 * C::VSTR + 32 * kb + 16 * j);
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][j], oacc[d], 0, 0, 0);
        }

    if (!LAST) {
      if (t + 2 < n_tiles) store_k(t & 1);
      store_v((t + 1) & 1);
      __syncthreads();
#pragma unroll
      for (int kb = 0; kb < C::KBLK; ++kb) scur[kb] = snext[kb];
    }
  };

  for (int t = 0; t + 1 < n_tiles; ++t) iteration(t, std::false_type{});
  if (n_tiles > 0) iteration(n_tiles - 1, std::true_type{});

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
}

}  // namespace

int launch_attn_fwd_bf16(const FwdArgs& a, int D, hipStream_t stream) {
  const int n_qb = (a.Nq + 127) / 128;
  const long long grid = (long long)n_qb * a.B * a.H;
  if (grid > 0x7fffffffLL) return -8;
  if (D == 128) {
    attn_fwd_bf16_kernel<128><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(a);
  } else {
    attn_fwd_bf16_kernel<64><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace attn89
