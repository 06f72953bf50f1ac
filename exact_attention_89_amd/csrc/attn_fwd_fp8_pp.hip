// attn_fwd_fp8_pp.hip -- the FP8 fused attention forward for gfx950 in 8-wave
// "ping-pong" workgroups (chosen for head dimension 128 and grids that fill the GPU;
// head dimension 64 on request).
//
// Same function and arithmetic as attn_fwd_fp8.hip (E4M3 Q, K, V with one descale
// per tensor; both products on v_mfma_f32_32x32x64_f8f6f4; P rounded to E4M3 as
// 2^kPShift p; bf16 O, fp32 LSE; page "Fused Multi-Head Attention", quantization
// item; page "Attention softmax fusion", sections "What fused has to mean" and
// "The tile loop"), with the work split of attn_fwd_bf16_pp.hip: one workgroup = 8
// waves = 256 query rows of one (batch, head), all 8 waves sharing each 64-key K/V
// tile in LDS; waves w and w+4 share a SIMD and form two groups, G0 = waves 0-3 and
// G1 = waves 4-7, half a tile apart, so one group's matrix phase (P.V of the
// previous tile and Q.K^T of this one, 8 FP8 MFMAs) runs while the other group
// computes its softmax.  The FP8 softmax (exponentials, sums, maxima and E4M3 packs of
// 32 scores per lane) takes longer than the FP8 matrix phase, so here the vector work
// sets the pace and the matrix phase hides behind it.
//
//   phase   G0                          G1
//   0       S(0) = K(0) Q^T             (loads K(1))
//   1       softmax(0) -> P(0)          S(0)
//   2       O += V(0) P(0); S(1)        softmax(0)
//   3       softmax(1)                  O += V(0) P(0); S(1)
//   ...     (every phase ends with a workgroup barrier)
//
// Data movement: G1 moves K tiles global -> LDS (buffer_load ... lds, 8 KiB per tile);
// G0 loads V tiles into registers and writes them as V^T in the P byte order
// (attn_fp8_tiles.hpp) during its softmax phase.  Both double buffered, requested two
// phases before first use; 32 KiB of LDS.
#include <type_traits>

#include "attn_fp8_tiles.hpp"
#include "launch.hpp"

namespace attn89 {
namespace {

template <int D>
struct CfgP8 {
  static constexpr int BR = 256;                 // query rows per workgroup
  static constexpr int BC = 64;                  // keys per tile
  static constexpr int ROWB = D;                 // bytes per K row
  static constexpr int TILE = BC * D;            // bytes per K tile (and per V^T tile)
  static constexpr int VTROWB = BC;              // bytes per V^T row
  static constexpr int KDMA = TILE / 1024 / 4;   // 1 KiB K loads per G1 wave per tile
  static constexpr int V_UNITS = (BC / 4) * (D / 8);  // G0 threads staging V (4 keys x 8 dims)
  static constexpr int DSTEPS = D / 64;          // k-steps of S^T = K Q^T
  static constexpr int DBLK = D / 32;            // 32-dimension blocks of O^T
  static constexpr int LDS = 4 * TILE;           // K double buffer, V^T double buffer
  static constexpr int VT0 = 2 * TILE;           // offset of the V^T buffers
  static_assert(V_UNITS <= 256, "V staging must fit in group 0");
};

__device__ __forceinline__ void phase_barrier8() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void wait_vm0_8() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Matrix phase of NM MFMAs, each fed by two 16-byte fragment reads: the reads of the
// first two MFMAs go first, then two reads after every MFMA, so every fragment is
// requested two MFMAs (128 cycles) before its use.
template <int NM>
__device__ __forceinline__ void schedule_fp8_phase() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // LDS reads
#pragma unroll
  for (int i = 0; i < NM - 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

template <int D, bool PRE>
__global__ __launch_bounds__(512) void attn_fwd_fp8_pp_kernel(FwdArgs p, float v_descale) {
  using C = CfgP8<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS];
  lds_u8* const lds = (lds_u8*)smem;

  const int tid = threadIdx.x;
  // wave-uniform values in scalar registers: branches on them are real branches and a
  // barrier never sits in a lane-masked region
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;     // 0: G0 (stages V), 1: G1 (moves K)
  const int wg = wave & 3;
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int lg = lane >> 5;

  // heaviest query blocks first; consecutive workgroups take different (b, h)
  const int BH = p.B * p.H;
  const int n_qb = (p.Nq + C::BR - 1) / C::BR;
  const int qb = n_qb - 1 - (int)blockIdx.x / BH;
  const int bh = (int)blockIdx.x % BH;
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

  // ---- K (G1): global -> LDS without registers (swizzled row-major) ----
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (unsigned)L * D);
  unsigned koff[C::KDMA];
#pragma unroll
  for (int n = 0; n < C::KDMA; ++n) {
    const int byte = (wg * C::KDMA + n) * 1024 + 16 * lane;
    const int row = byte / C::ROWB;
    const int ch = ((byte % C::ROWB) / 16) ^ kswz8<D>(row);
    koff[n] = (unsigned)row * D + 16 * ch;
  }
  auto load_k = [&](int t, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < C::KDMA; ++n)
      buffer_load16_to_lds(krs, (lds_void*)(lds + stage * C::TILE + (wg * C::KDMA + n) * 1024),
                           koff[n], t * C::BC * D);
  };

  // ---- V (G0): global -> registers -> LDS as V^T in the P byte order ----
  // Thread (kg, dg) of G0 holds keys 4kg .. 4kg+3 x dimensions 8dg .. 8dg+7 and writes
  // 8 dwords (one per dimension, the 4 keys' bytes): dword g of logical chunk 2h + kb
  // of the row, kb = kg/8, g = (kg%8)/2, h = kg%2.
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, (unsigned)L * D);
  const bool v_owner = tid < C::V_UNITS;   // used by G0 only
  const int vkg = tid % (C::BC / 4), vdg = (tid / (C::BC / 4)) % (D / 8);
  const unsigned vgoff = (unsigned)(4 * vkg) * D + 8 * vdg;
  unsigned vwoff[2];
  const int vchunk = 2 * (vkg & 1) + (vkg >> 3);
  const int vdw = (vkg >> 1) & 3;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int d = 8 * vdg + 4 * i;
    vwoff[i] = d * C::VTROWB + ((vchunk ^ vtswz8(d)) * 16) + 4 * vdw;
  }
  u32x2 vreg[4];
  auto load_v = [&](int t) __attribute__((always_inline)) {
    if (v_owner) {
#pragma unroll
      for (int r = 0; r < 4; ++r) vreg[r] = buffer_load8_so(vrs, vgoff + r * D, t * C::BC * D);
    }
  };
  auto store_v = [&](int buf) __attribute__((always_inline)) {
    if (v_owner) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x4 d4 = transpose4x4_bytes(vreg[0][i], vreg[1][i], vreg[2][i], vreg[3][i]);
#pragma unroll
        for (int x = 0; x < 4; ++x)
          *(__attribute__((address_space(3))) unsigned*)(
              lds + C::VT0 + buf * C::TILE + vwoff[i] + x * C::VTROWB) = d4[x];
      }
    }
  };

  // ---- fragment read offsets ----
  unsigned kro[C::DSTEPS][2];
#pragma unroll
  for (int s = 0; s < C::DSTEPS; ++s)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      kro[s][c] = lq * C::ROWB + (((4 * s + 2 * lg + c) ^ kswz8<D>(lq)) * 16);
  unsigned vro[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) vro[c] = lq * C::VTROWB + (((2 * lg + c) ^ vtswz8(lq)) * 16);

  // ---- running state: one query per lane ----
  f32x16 oacc[C::DBLK];
#pragma unroll
  for (int d = 0; d < C::DBLK; ++d) oacc[d] = (f32x16){};
  f32x16 sacc[2];   // S(t), from its matrix phase to its softmax phase
  i32x8 pf;         // P(t) in E4M3, from its softmax phase to the next matrix phase
  float m_run = kNegInf;
  float l_run = 0.f;
  const float c_exp = p.c_exp;

  auto qk = [&](int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < C::DSTEPS; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const lds_u8* base = lds + stage * C::TILE + kb * 32 * C::ROWB;
        const i32x8 a = join32(lds_load<u32x4>(base, kro[s][0]), lds_load<u32x4>(base, kro[s][1]));
        sacc[kb] = mfma_fp8(a, qf[s], s == 0 ? (f32x16){} : sacc[kb]);
      }
  };
  auto pv = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < C::DBLK; ++d) {
      const lds_u8* base = lds + C::VT0 + buf * C::TILE + d * 32 * C::VTROWB;
      const i32x8 va = join32(lds_load<u32x4>(base, vro[0]), lds_load<u32x4>(base, vro[1]));
      oacc[d] = mfma_fp8(va, pf, oacc[d]);
    }
  };

  // softmax of tile t: mask, row maxima -> exponent reference, lazy correction of O
  // and l, P = 2^kPShift exp2(s*c - m) packed to E4M3 in the B-operand byte order
  auto softmax = [&](int t) __attribute__((always_inline)) {
    const int j0 = t * C::BC;
    if (PRE || (j0 + C::BC > L) || (p.causal && j0 + C::BC - 1 > qw)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + kb * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
          const bool ok = (key < L) & (!p.causal | (key <= qrow));
          const float x = PRE ? sacc[kb][r] * p.c_pre : sacc[kb][r];
          sacc[kb][r] = ok ? x : kNegInf;
        }
    }
    // guard: a row with no valid key so far keeps m = -inf and uses 0 as its
    // exponent reference, so no -inf - (-inf) is ever formed
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = max_with_partner(mx) * c_exp;
    const bool move = mx > m_run + kSlack8;
    const float m_new = move ? mx : m_run;
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    if (__any(move)) {
      const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
    }
    m_run = m_new;
    const float m_sh = m_use - kPShift;
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        pf[4 * kb + w] = exp2_pack_e4m3(sacc[kb][4 * w], sacc[kb][4 * w + 1],
                                        sacc[kb][4 * w + 2], sacc[kb][4 * w + 3], c_exp, m_sh,
                                        lsum);
    l_run += lsum;
  };

  auto epilogue = [&]() __attribute__((always_inline)) {
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
  };

  // One tile period of group G; PAR = t & 1 selects the buffers at compile time.
  //   matrix phase:  O += V(t-1) P(t-1) (t > 0), S(t) = K(t) Q^T
  //   softmax phase: P(t); G0 writes V(t) to V^T buffer PAR and requests V(t+1),
  //                  G1 requests K(t+2) into K buffer PAR
  auto period = [&](const int t, auto grp_tag, auto par_tag, auto first_tag)
                    __attribute__((always_inline)) {
    constexpr int G = decltype(grp_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    constexpr bool FIRST = decltype(first_tag)::value;
    __builtin_amdgcn_s_setprio(1);
    if (!FIRST) pv(PAR ^ 1);
    qk(PAR);
    schedule_fp8_phase<FIRST ? 2 * C::DSTEPS : 2 * C::DSTEPS + C::DBLK>();
    if (G == 1) wait_vm0_8();   // K(t+1) has landed: it is read after the barrier
    phase_barrier8();
    __builtin_amdgcn_s_setprio(0);
    softmax(t);
    if (G == 0) {
      store_v(PAR);
      if (t + 1 < n_tiles) load_v(t + 1);
    } else {
      if (t + 2 < n_tiles) load_k(t + 2, PAR);
    }
    phase_barrier8();
  };

  // the whole key loop of one group as straight-line code of its own (one shared body
  // would merge the two groups' register states)
  auto run_group = [&](auto grp_tag) __attribute__((always_inline)) {
    constexpr int G = decltype(grp_tag)::value;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    if (n_tiles > 0) {
      if (G == 1) load_k(0, 0);
      else load_v(0);
    }
    if (G == 1) wait_vm0_8();
    phase_barrier8();
    if (n_tiles > 0) {
      if (G == 1) {
        // G1 starts one phase late; meanwhile it requests K(1)
        if (n_tiles > 1) load_k(1, 1);
        phase_barrier8();
      }
      period(0, grp_tag, I0{}, std::true_type{});
      int t = 1;
      for (; t + 1 < n_tiles; t += 2) {
        period(t, grp_tag, I1{}, std::false_type{});
        period(t + 1, grp_tag, I0{}, std::false_type{});
      }
      if (t < n_tiles) period(t, grp_tag, I1{}, std::false_type{});
      // last matrix phase: O += V(n-1) P(n-1)
      __builtin_amdgcn_s_setprio(1);
      if ((n_tiles - 1) & 1) pv(1);
      else pv(0);
      __builtin_amdgcn_s_setprio(0);
      // G0 ends one phase early; it meets G1's last softmax barrier
      if (G == 0) phase_barrier8();
    }
    epilogue();
  };

  if (grp == 0) run_group(std::integral_constant<int, 0>{});
  else run_group(std::integral_constant<int, 1>{});
}

}  // namespace

int launch_attn_fwd_fp8_pp(const FwdArgs& a, int D, float v_descale, hipStream_t stream) {
  const int n_qb = (a.Nq + 255) / 256;
  const long long grid = (long long)n_qb * a.B * a.H;
  if (grid > 0x7fffffffLL) return -8;
  const dim3 g((unsigned)grid), blk(512);
  if (D == 128) {
    if (a.pre_scale)
      attn_fwd_fp8_pp_kernel<128, true><<<g, blk, 0, stream>>>(a, v_descale);
    else
      attn_fwd_fp8_pp_kernel<128, false><<<g, blk, 0, stream>>>(a, v_descale);
  } else {
    if (a.pre_scale)
      attn_fwd_fp8_pp_kernel<64, true><<<g, blk, 0, stream>>>(a, v_descale);
    else
      attn_fwd_fp8_pp_kernel<64, false><<<g, blk, 0, stream>>>(a, v_descale);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace attn89
