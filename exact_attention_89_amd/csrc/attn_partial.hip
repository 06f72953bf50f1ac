// attn_partial.hip -- partial fusion: Q K^T and the softmax in one launch, the
// probabilities written to device memory, P V in a second launch.
//
// Page "Attention softmax fusion", section "What fused has to mean" (the case where
// only one of the two boundaries is fused): each score tile stays on chip from the
// Q K^T contraction until it is a normalised probability, yet P is still stored,
// since the P V launch is separate and can only get it from device memory.  About
// half of the score-sized traffic of the three-launch form remains, and an Nq x Nk
// tensor is still materialised.
//
// Launch 1 (this file), one workgroup = 4 waves = 128 query rows:
//   pass 1  for every key tile: S = K Q^T (MFMA, fp32), mask, and the online row
//           statistics m, l (the correction exp2(m_old - m_new) on l when the
//           maximum rises; fully masked rows keep m = -inf, reference 0)
//   pass 2  for every key tile again: S = K Q^T, mask, P = exp2(s c - m) / l in
//           registers, rounded to bf16 and stored row-major into P[q][key]; tiles
//           no row of the block can see are stored as zeros, so the whole row of P
//           (ld = Nk rounded up to 64 columns) is defined
//   LSE = ln2 (m + log2 l)
// Launch 2: launch_pv (attn_materialized.hip), O = P V.
//
// The score layout (transposed scores, lane = query, keys in the bits-2-and-3-swapped
// order) and the swizzled K tiles are those of attn_bf16_tiles.hpp: register r of lane
// l holds key 16*(r/8) + 8*(l/32) + r%8 of its 32-key block, so 8 consecutive
// registers are 8 consecutive keys, one 16-byte store of P.

#include <type_traits>

#include "attn_bf16_tiles.hpp"
#include "launch.hpp"

namespace attn89 {
namespace {

template <int D>
struct PCfg {
  static constexpr int BR = 128;
  static constexpr int BC = 64;
  static constexpr int ROWB = D * 2;
  static constexpr int TILE = BC * ROWB;
  static constexpr int DMA = TILE / 1024 / 4;
  static constexpr int DSTEPS = D / 16;
  static constexpr int KBLK = BC / 32;
  static constexpr int LDS = 2 * TILE;
};

template <int D, bool PRE>
__global__ __launch_bounds__(256, 2) void qk_softmax_kernel(FwdArgs p, int ld,
                                                           unsigned short* P) {
  using C = PCfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS];
  lds_u8* const lds = (lds_u8*)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int lg = lane >> 5;

  const int BH = p.B * p.H;
  const int n_qb = (p.Nq + C::BR - 1) / C::BR;
  const int qb = n_qb - 1 - (int)blockIdx.x / BH;
  const int bh = (int)blockIdx.x % BH;
  const int b = bh / p.H;

  const unsigned short* qp = (const unsigned short*)p.q + (size_t)bh * p.Nq * D;
  const unsigned short* kp = (const unsigned short*)p.k + (size_t)bh * p.Nk * D;
  unsigned short* pp = P + (size_t)bh * p.Nq * ld;
  float* lsep = p.lse + (size_t)bh * p.Nq;

  const int L = clamp_len(p.kv_lens, b, p.Nk);
  const int q0 = qb * C::BR;
  const int q_hi = min(q0 + C::BR, p.Nq);
  const int kv_end = p.causal ? min(L, q_hi) : L;
  const int n_tiles = (kv_end + C::BC - 1) / C::BC;
  const int n_out = ld / C::BC;                       // tiles of the P row
  const int qw = q0 + wave * 32;
  const int qrow = qw + lq;

  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qp, (unsigned)p.Nq * D * 2);
  bf16x8 qf[C::DSTEPS];
#pragma unroll
  for (int s = 0; s < C::DSTEPS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8,
                               buffer_load16(qrs, ((unsigned)qrow * D + 16 * s + 8 * lg) * 2));

  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (unsigned)L * D * 2);
  unsigned koff[C::DMA];
#pragma unroll
  for (int n = 0; n < C::DMA; ++n) {
    const int byte = (wave * C::DMA + n) * 1024 + 16 * lane;
    const int row = byte / C::ROWB;
    const int ch = ((byte % C::ROWB) / 16) ^ kswz<D>(row);
    koff[n] = ((unsigned)row * D + 8 * ch) * 2;
  }
  auto load_k = [&](int t, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < C::DMA; ++n)
      buffer_load16_to_lds(krs, (lds_void*)(lds + stage * C::TILE + (wave * C::DMA + n) * 1024),
                           koff[n], t * C::BC * D * 2);
  };
  const int krow = swap_bits23(lq);
  unsigned kro[C::DSTEPS];
#pragma unroll
  for (int s = 0; s < C::DSTEPS; ++s)
    kro[s] = krow * C::ROWB + (((2 * s + lg) ^ kswz<D>(krow)) * 16);

  auto qk = [&](int stage, f32x16* sacc) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < C::DSTEPS; ++s)
#pragma unroll
      for (int kb = 0; kb < C::KBLK; ++kb) {
        const bf16x8 a = lds_load<bf16x8>(lds + stage * C::TILE + kb * 32 * C::ROWB, kro[s]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            a, qf[s], s == 0 ? (f32x16){} : sacc[kb], 0, 0, 0);
      }
  };
  auto mask = [&](int t, f32x16* sacc) __attribute__((always_inline)) {
    const int j0 = t * C::BC;
    if (PRE || (j0 + C::BC > L) || (p.causal && j0 + C::BC - 1 > qw)) {
#pragma unroll
      for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + kb * 32 + 16 * (r >> 3) + 8 * lg + (r & 7);
          const bool ok = (key < L) & (!p.causal | (key <= qrow));
          const float x = PRE ? sacc[kb][r] * p.c_pre : sacc[kb][r];
          sacc[kb][r] = ok ? x : kNegInf;
        }
    }
  };
  const float c_exp = p.c_exp;

  // ---- pass 1: row statistics ----
  float m_run = kNegInf;   // running maximum (log2 domain)
  float l_run = 0.f;       // this lane's part of the sum, against the reference of m_run
  auto stats = [&](const int t, auto par_tag, auto last_tag) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    constexpr bool LAST = decltype(last_tag)::value;
    if (!LAST) load_k(t + 1, PAR ^ 1);
    f32x16 sacc[C::KBLK];
    qk(PAR, sacc);
    mask(t, sacc);
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = max_with_partner(mx) * c_exp;
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float m_old = (m_run == kNegInf) ? 0.f : m_run;
    float s = l_run * __builtin_amdgcn_exp2f(m_old - m_use);
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], c_exp, -m_use));
    l_run = s;
    m_run = m_new;
    if (!LAST) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): K(t+1) in LDS
      __syncthreads();
    }
  };

  // ---- pass 2: P = exp2(s c - m) / l, stored as bf16 ----
  float m_fin = kNegInf, inv = 0.f;
  unsigned short* prow = pp + (size_t)qrow * ld;
  auto store_tile = [&](int t, const u32x4 (&w)[C::KBLK][2]) __attribute__((always_inline)) {
    if (qrow < p.Nq) {
#pragma unroll
      for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          *(u32x4*)(prow + t * C::BC + kb * 32 + 16 * j + 8 * lg) = w[kb][j];
    }
  };
  auto emit = [&](const int t, auto par_tag, auto last_tag) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    constexpr bool LAST = decltype(last_tag)::value;
    if (!LAST) load_k(t + 1, PAR ^ 1);
    f32x16 sacc[C::KBLK];
    qk(PAR, sacc);
    mask(t, sacc);
    const float m_use = (m_fin == kNegInf) ? 0.f : m_fin;
    u32x4 w[C::KBLK][2];
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float e0 = __builtin_amdgcn_exp2f(
              __builtin_fmaf(sacc[kb][8 * j + 2 * x], c_exp, -m_use)) * inv;
          const float e1 = __builtin_amdgcn_exp2f(
              __builtin_fmaf(sacc[kb][8 * j + 2 * x + 1], c_exp, -m_use)) * inv;
          w[kb][j][x] = pack_bf16x2(e0, e1);
        }
    store_tile(t, w);
    if (!LAST) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto run_tiles = [&](auto body) __attribute__((always_inline)) {
    if (n_tiles > 0) {
      load_k(0, 0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      int t = 0;
      for (; t + 2 < n_tiles; t += 2) {
        body(t, I0{}, std::false_type{});
        body(t + 1, I1{}, std::false_type{});
      }
      if (t + 1 < n_tiles) {
        body(t, I0{}, std::false_type{});
        body(t + 1, I1{}, std::true_type{});
      } else {
        body(t, I0{}, std::true_type{});
      }
    }
  };

  run_tiles(stats);
  const float l_tot = sum_with_partner(l_run);
  m_fin = m_run;
  inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  __syncthreads();   // every wave is done with the K buffers of pass 1
  run_tiles(emit);
  // tiles past the block's last visible key: zeros
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const u32x4 zw[C::KBLK][2] = {{zero4, zero4}, {zero4, zero4}};
  for (int t = n_tiles; t < n_out; ++t) store_tile(t, zw);

  if (qrow < p.Nq && lg == 0)
    lsep[qrow] = l_tot > 0.f ? (m_fin + __builtin_amdgcn_logf(l_tot)) * kLn2 : kNegInf;
}

}  // namespace

int launch_attn_partial(const FwdArgs& a, int D, int ld, unsigned short* P,
                        hipStream_t stream) {
  const int n_qb = (a.Nq + 127) / 128;
  const long long grid = (long long)n_qb * a.B * a.H;
  if (grid > 0x7fffffffLL) return -8;
  const dim3 g((unsigned)grid), blk(256);
  if (D == 128) {
    if (a.pre_scale)
      qk_softmax_kernel<128, true><<<g, blk, 0, stream>>>(a, ld, P);
    else
      qk_softmax_kernel<128, false><<<g, blk, 0, stream>>>(a, ld, P);
  } else {
    if (a.pre_scale)
      qk_softmax_kernel<64, true><<<g, blk, 0, stream>>>(a, ld, P);
    else
      qk_softmax_kernel<64, false><<<g, blk, 0, stream>>>(a, ld, P);
  }
  if (hipGetLastError() != hipSuccess) return -7;
  return launch_pv(a, D, ld, P, stream);
}

}  // namespace attn89
