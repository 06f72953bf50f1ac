// attn_fwd_fp8.hip -- the fused attention forward for gfx950 on FP8 inputs: Q, K, V
// as OCP E4M3 codes with one dequantisation factor per tensor, both products on the
// FP8 matrix cores (v_mfma_f32_32x32x64_f8f6f4, fp32 accumulation), bf16 O, fp32 LSE.
//
// The page "Fused Multi-Head Attention" (quantization item of the section on how
// fused attention combines with other techniques) names FP8 data for the matrix
// products of a fused kernel.  Everything else is the fused forward of
// attn_fwd_bf16_4w.hip: scores, mask, online softmax with the exp(m_old - m_new)
// correction and the P.V product stay in the workgroup (page "Attention softmax
// fusion", sections "What fused has to mean" and "The tile loop").
//
// Arithmetic.  Scores are s = (scale * q_descale * k_descale) * sum_d q8 k8; the
// products of two E4M3 values are exact in fp32 and are summed in fp32.  The
// probabilities enter the second product as E4M3: p' = 2^kPShift * exp2(s*c - m),
// rounded to nearest even by v_cvt_pk_fp8_f32.  The shift keeps p' in E4M3's
// normal range (relative rounding error <= 2^-4) down to p = 2^-12, and with the
// exponent reference allowed to lag the row maximum by at most kSlack8 (log2 units)
// p' <= 2^(kPShift + kSlack8) = 256 < 448, the largest E4M3 value.  The normaliser
// l sums the unrounded p' in fp32.  O = v_descale * (sum p'_rounded v8) / l, LSE =
// ln2 * (m + log2 l - kPShift).
//
// Layout (one workgroup = 4 waves = 128 query rows of one (batch, head); key tiles
// of 64).  Scores are computed transposed, S^T = K Q^T: A = 32 keys x 64 dimensions
// of K (from LDS), B = 64 dimensions x 32 queries of Q^T (in VGPRs for the whole
// loop).  Lane l feeds row / column l%32 of its operand and 32 consecutive bytes of
// the reduction dimension (half l/32); the hardware's order inside the reduction
// does not matter as long as A and B use the same one, which they do.  The score
// accumulator of 32 keys x 32 queries leaves register r of lane l with key
// 8*(r/4) + 4*(l/32) + r%4 and query l%32, so the 64 P values of a lane (two 32-key
// blocks) are exactly the 32 bytes one B operand of O^T = V^T P^T needs: byte
// 16*kb + r of lane half h is key 32*kb + 8*(r/4) + 4*h + r%4.  The A operand of
// O^T = V^T P^T (one dimension per lane, its 64 keys in that byte order) is read from
// the row-major V tile with four transposing LDS reads (ds_read_b64_tr_b8), whose lane
// addresses pick the keys in the P byte order.
//
// Data movement.  K and V tiles both go global -> LDS by buffer_load ... lds
// (row-major, 16-byte chunks XOR-swizzled by row), double buffered, no registers and
// no vector instructions; the key loop is unrolled by two so every LDS offset is an
// immediate, and each buffer is an LDS array of its own so that no fragment read waits
// for the next tile's loads.  (Staging V through registers and transposing it with
// byte permutes cost 16 vector instructions per tile and thread, in a kernel whose
// vector unit is the bottleneck; the transposing reads replaced them: +8 % at B=1
// H=32 N=8192 causal.)
#include <type_traits>

#include "attn_fp8_tiles.hpp"
#include "launch.hpp"
#include "mfma_schedule.hpp"

namespace attn89 {
namespace {

template <int D>
struct Cfg8 {
  static constexpr int BR = 128;                 // query rows per workgroup
  static constexpr int BC = 64;                  // keys per tile
  static constexpr int NT = 256;                 // threads per workgroup
  static constexpr int ROWB = D;                 // bytes per K row
  static constexpr int TILE = BC * D;            // bytes per K (or V) tile
  static constexpr int DMA = TILE / 1024 / 4;    // 1 KiB K loads per wave per tile
  static constexpr int DSTEPS = D / 64;          // k-steps of S^T = K Q^T
  static constexpr int DBLK = D / 32;            // 32-dimension blocks of O^T
};

// PRE: scale <= 0, scores are scaled before they are masked.
template <int D, bool PRE>
__global__ __launch_bounds__(256, 2) void attn_fwd_fp8_kernel(FwdArgs p, float v_descale) {
  using C = Cfg8<D>;
  // K and V double buffers, each buffer an LDS array of its own: a fragment read of one
  // buffer while a DMA into the other is in flight must not look like a possible
  // overlap to the compiler, which would wait for the outstanding loads first
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
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int lg = lane >> 5;

  // Schedule (as in the bf16 ping-pong kernel): workgroup i runs on XCD i mod 8.
  // Non-causal with B*H a multiple of 8: each XCD takes its heads one at a time; causal
  // with B*H a multiple of 16: two at a time, the two heads' blocks interleaved, heaviest
  // (last) first, so every CU ends with the same number of key tiles and the blocks that
  // run together share K/V tiles in L2 (half the device-memory reads of the order below
  // at B=1 H=32 N=8192, same time); otherwise heaviest blocks first, consecutive
  // workgroups taking different (b, h).
  const int BH = p.B * p.H;
  const int n_qb = (p.Nq + C::BR - 1) / C::BR;
  int qb, bh;
  if (!p.causal && BH % 8 == 0) {
    const int x = (int)blockIdx.x % 8, slot = (int)blockIdx.x / 8;
    bh = x + 8 * (slot / n_qb);
    qb = n_qb - 1 - slot % n_qb;
  } else if (BH % 16 == 0) {
    const int x = (int)blockIdx.x & 7, slot = (int)blockIdx.x >> 3;
    const int pair = slot / (2 * n_qb), r = slot - pair * 2 * n_qb;
    bh = x + 8 * (2 * pair + (r & 1));
    qb = n_qb - 1 - (r >> 1);
  } else {
    qb = n_qb - 1 - (int)blockIdx.x / BH;
    bh = (int)blockIdx.x % BH;
  }
  const int b = bh / p.H;

  const unsigned char* qp = (const unsigned char*)p.q + (size_t)bh * p.Nq * D;
  const unsigned char* kp = (const unsigned char*)p.k + (size_t)bh * p.Nk * D;
  const unsigned char* vp = (const unsigned char*)p.v + (size_t)bh * p.Nk * D;
  unsigned short* op = (unsigned short*)p.o + (size_t)bh * p.Nq * D;
  float* lsep = p.lse + (size_t)bh * p.Nq;

  const int L = clamp_len(p.kv_lens, b, p.Nk);
  const int q0 = qb * C::BR;
  const int q_hi = min(q0 + C::BR, p.Nq);
  const int kv_end = p.causal ? min(L, q_hi) : L;
  const int n_tiles = (kv_end + C::BC - 1) / C::BC;
  // leading tiles whose keys are all visible to every row of the block
  const int n_full = PRE ? 0 : min(L, p.causal ? q0 + 1 : L) / C::BC;
  const int qw = q0 + wave * 32;
  const int qrow = qw + lq;

  // ---- Q fragments: dimensions 64s + 32*lg .. + 32 of query qrow (zeros past Nq) ----
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qp, (unsigned)p.Nq * D);
  i32x8 qf[C::DSTEPS];
#pragma unroll
  for (int s = 0; s < C::DSTEPS; ++s) {
    const unsigned off = (unsigned)qrow * D + 64 * s + 32 * lg;
    qf[s] = join32(buffer_load16(qrs, off), buffer_load16(qrs, off + 16));
  }

  // ---- K: global -> LDS without registers (swizzled row-major) ----
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (unsigned)L * D);
  unsigned koff[C::DMA];
#pragma unroll
  for (int n = 0; n < C::DMA; ++n) {
    const int byte = (wave * C::DMA + n) * 1024 + 16 * lane;
    const int row = byte / C::ROWB;
    const int ch = ((byte % C::ROWB) / 16) ^ kswz8<D>(row);
    koff[n] = (unsigned)row * D + 16 * ch;
  }
  auto load_k = [&](int t, int stage) {
#pragma unroll
    for (int n = 0; n < C::DMA; ++n)
      buffer_load16_to_lds(krs, (lds_void*)(kbuf(stage) + (wave * C::DMA + n) * 1024),
                           koff[n], t * C::BC * D);
  };

  // ---- V: global -> LDS without registers, row-major like K ----
  // The P.V operand (V^T: 32 dimensions x 64 keys per lane group, in the P byte order)
  // is read back with the transposing ds_read_b64_tr_b8: in each group of 16 lanes, the
  // lane 16g + 8h + j receives, as byte m of its 8, byte j of the 8 bytes at the address
  // of lane 16g + h + 2m.  So the lane that holds position i of its group addresses, in
  // read q, key 16q + 8(m/4) + 4(g/2) + m%4 (m = i/2: the key whose P byte sits at
  // position 8q + m of lane half g/2) at dimensions 16(g%2) + 8(i%2) .. + 8 of the
  // 32-dimension block: four reads give a lane its 32 operand bytes.
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, (unsigned)L * D);
  auto load_v = [&](int t, int stage) {
#pragma unroll
    for (int n = 0; n < C::DMA; ++n)
      buffer_load16_to_lds(vrs,
                           (lds_void*)(vbuf(stage) + (wave * C::DMA + n) * 1024),
                           koff[n], t * C::BC * D);
  };
  unsigned vtr[C::DBLK];   // read q of 32-dimension block d: vtr[d] + 16 q rows
  {
    const int gi = lane & 15, gg = lane >> 4, m = gi >> 1;
    const int key = 8 * (m >> 2) + 4 * (gg >> 1) + (m & 3);   // + 16 q (same swizzle)
#pragma unroll
    for (int d = 0; d < C::DBLK; ++d)
      vtr[d] = key * C::ROWB + (((2 * d + (gg & 1)) ^ kswz8<D>(key)) * 16) + 8 * (gi & 1);
  }

  // ---- fragment read offsets ----
  // K: row lq of each 32-key block, logical chunks 4s + 2lg and 4s + 2lg + 1
  unsigned kro[C::DSTEPS][2];
#pragma unroll
  for (int s = 0; s < C::DSTEPS; ++s)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      kro[s][c] = lq * C::ROWB + (((4 * s + 2 * lg + c) ^ kswz8<D>(lq)) * 16);

  auto qk = [&](int stage, f32x16* sacc) {
#pragma unroll
    for (int s = 0; s < C::DSTEPS; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const lds_u8* base = kbuf(stage) + kb * 32 * C::ROWB;
        const i32x8 a = join32(lds_load<u32x4>(base, kro[s][0]), lds_load<u32x4>(base, kro[s][1]));
        sacc[kb] = mfma_fp8(a, qf[s], s == 0 ? (f32x16){} : sacc[kb]);
      }
  };

  auto needs_mask = [&](int t) {
    const int j0 = t * C::BC;
    return PRE || (j0 + C::BC > L) || (p.causal && j0 + C::BC - 1 > qw);
  };
  auto apply_mask = [&](int t, f32x16* sacc) {
    // key j0 + off of this lane is visible iff off < lim (kv_len and causal bounds)
    const int lim = min(L, p.causal ? qrow + 1 : L) - t * C::BC - 4 * lg;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
        const float x = PRE ? sacc[kb][r] * p.c_pre : sacc[kb][r];
        sacc[kb][r] = off < lim ? x : kNegInf;
      }
  };

  f32x16 oacc[C::DBLK];
#pragma unroll
  for (int d = 0; d < C::DBLK; ++d) oacc[d] = (f32x16){};
  float m_run = kNegInf;
  float l_run = 0.f;
  const float c_exp = p.c_exp;

  auto iteration = [&](const int t, auto par_tag, auto last_tag, auto mask_tag) {
    constexpr int PAR = decltype(par_tag)::value;
    constexpr bool LAST = decltype(last_tag)::value;
    constexpr bool MASKED = decltype(mask_tag)::value;
    if (!LAST) {
      load_k(t + 1, PAR ^ 1);
      load_v(t + 1, PAR ^ 1);
    }
    f32x16 scur[2];
    qk(PAR, scur);
    schedule_mfma_run<C::DSTEPS * 2, 2, LAST ? 0 : 2 * C::DMA, 2>();
    if (MASKED && needs_mask(t)) apply_mask(t, scur);
    // row maximum and exponent reference (guard: a row without a valid key so far
    // keeps m = -inf and uses 0 as its reference)
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, scur[kb][r]);
    mx = max_with_partner(mx) * c_exp;
    const bool move = mx > m_run + kSlack8;
    const float m_new = move ? mx : m_run;
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    if (__builtin_expect(__any(move), 0)) {
      const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
    }
    m_run = m_new;
    // p' = exp2(s*c - m + kPShift), packed to E4M3: byte 16kb + r <- register r of block kb
    const float m_sh = m_use - kPShift;
    i32x8 pf;
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pf[4 * kb + w] = exp2_pack_e4m3(scur[kb][4 * w], scur[kb][4 * w + 1], scur[kb][4 * w + 2],
                                        scur[kb][4 * w + 3], c_exp, m_sh, lsum);
      }
    l_run += lsum;
    // O^T += V^T P^T
#pragma unroll
    for (int d = 0; d < C::DBLK; ++d) {
      const lds_u8* base = vbuf(PAR) + vtr[d];
      const i32x8 va = join_tr8(lds_tr8(base), lds_tr8(base + 16 * C::ROWB),
                                lds_tr8(base + 32 * C::ROWB), lds_tr8(base + 48 * C::ROWB));
      oacc[d] = mfma_fp8(va, pf, oacc[d]);
    }
    schedule_mfma_run<C::DBLK, 4, 0, 2>();
    if (!LAST) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's K(t+1), V(t+1) landed
      __syncthreads();
    }
  };

  if (n_tiles > 0) {
    load_v(0, 0);
    load_k(0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): also drains the Q fragments
  __syncthreads();
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  int t = 0;
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

  // ---- epilogue: O = v_descale * a / l (0 without a valid key), LSE ----
  const float l_tot = sum_with_partner(l_run);
  if (qrow < p.Nq) {
    const float inv = l_tot > 0.f ? v_descale / l_tot : 0.f;
    unsigned short* orow = op + (size_t)qrow * D;
#pragma unroll
    for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 w = {pack_bf16x2(oacc[d][4 * a + 0] * inv, oacc[d][4 * a + 1] * inv),
                   pack_bf16x2(oacc[d][4 * a + 2] * inv, oacc[d][4 * a + 3] * inv)};
        *(u32x2*)(orow + d * 32 + 8 * a + 4 * lg) = w;
      }
    if (lg == 0)
      lsep[qrow] = l_tot > 0.f
                       ? (m_run + __builtin_amdgcn_logf(l_tot) - kPShift) * kLn2
                       : kNegInf;
  }
}

}  // namespace

int launch_attn_fwd_fp8(const FwdArgs& a, int D, float v_descale, hipStream_t stream) {
  const int n_qb = (a.Nq + 127) / 128;
  const long long grid = (long long)n_qb * a.B * a.H;
  if (grid > 0x7fffffffLL) return -8;
  const dim3 g((unsigned)grid), blk(256);
  if (D == 128) {
    if (a.pre_scale)
      attn_fwd_fp8_kernel<128, true><<<g, blk, 0, stream>>>(a, v_descale);
    else
      attn_fwd_fp8_kernel<128, false><<<g, blk, 0, stream>>>(a, v_descale);
  } else {
    if (a.pre_scale)
      attn_fwd_fp8_kernel<64, true><<<g, blk, 0, stream>>>(a, v_descale);
    else
      attn_fwd_fp8_kernel<64, false><<<g, blk, 0, stream>>>(a, v_descale);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace attn89
