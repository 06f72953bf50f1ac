// attn_materialized.hip -- the unfused three-launch attention, bf16.
//
// This is the pipeline a fused kernel replaces (page "Fused Multi-Head Attention":
// a score GEMM, a softmax kernel and a weighted-sum GEMM as separate launches; page
// "Attention softmax fusion", section "What fused has to mean").  Every launch
// writes its whole result to device memory and the next one reads it back:
//
//   qk_scores   S = scale * Q K^T, -inf where masked      (fp32, [B][H][Nq][ld])
//   softmax     P = exp(S - rowmax) / rowsum, LSE         (bf16, [B][H][Nq][ld])
//   pv          O = P V                                    (bf16, [B][H][Nq][D])
//
// ld is Nk rounded up to a multiple of 64; the padding columns hold S = -inf and
// P = 0.  It exists to measure the traffic the fused kernel avoids, so it makes no
// attempt to skip the masked half of a causal problem.  The two GEMMs use the same
// bf16 matrix instruction as the fused kernel.

#include "common.hpp"
#include "launch.hpp"

namespace attn89 {
namespace {

// ---- launch 1: S = scale * Q K^T ----------------------------------------------
// One workgroup = 4 waves = a 64x64 block of S; each wave a 32x32 block computed
// with v_mfma_f32_32x32x16_bf16, operands read directly from global memory
// (A = Q rows, B = K rows as columns).
template <int D>
__global__ __launch_bounds__(256) void qk_scores_kernel(FwdArgs p, float scale, int ld,
                                                        float* S) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lq = lane & 31, lg = lane >> 5;
  const int bh = blockIdx.z;
  const int b = bh / p.H;
  const int i0 = blockIdx.y * 64 + 32 * (wave >> 1);
  const int j0 = blockIdx.x * 64 + 32 * (wave & 1);
  const unsigned short* qp = (const unsigned short*)p.q + (size_t)bh * p.Nq * D;
  const unsigned short* kp = (const unsigned short*)p.k + (size_t)bh * p.Nk * D;
  const int L = clamp_len(p.kv_lens, b, p.Nk);

  const int qi = i0 + lq, kj = j0 + lq;
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    bf16x8 a = {}, bb = {};
    if (qi < p.Nq) a = *(const bf16x8*)(qp + (size_t)qi * D + 16 * s + 8 * lg);
    // keys past the sequence's length are never read (their scores are masked anyway)
    if (kj < L) bb = *(const bf16x8*)(kp + (size_t)kj * D + 16 * s + 8 * lg);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc, 0, 0, 0);
  }
  // accumulator register r of lane l: row 8*(r/4) + 4*(l/32) + r%4, column l%32
  float* Sh = S + (size_t)bh * p.Nq * ld;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = i0 + 8 * (r >> 2) + 4 * lg + (r & 3);
    if (i < p.Nq) {
      const bool ok = kj < L && (!p.causal || kj <= i);
      Sh[(size_t)i * ld + kj] = ok ? acc[r] * scale : kNegInf;
    }
  }
}

// ---- launch 2: row softmax ----------------------------------------------------
// One workgroup per row.  Pass 1 streams the row once and keeps a per-thread
// running (max, sum) pair, merged across the workgroup at the end; pass 2 streams
// it again and writes P.  Nothing sized by the row lives in registers.
__global__ __launch_bounds__(256) void softmax_rows_kernel(const float* S, unsigned short* P,
                                                           float* lse, int ld) {
  __shared__ float red_m[256];
  __shared__ float red_l[256];
  const size_t row = blockIdx.x;
  const float* s = S + row * ld;
  unsigned short* pr = P + row * ld;
  const int tid = threadIdx.x;

  float m = kNegInf, l = 0.f;
  for (int j = tid; j < ld; j += 256) {
    const float x = s[j];
    if (x > m) {
      l = l * __builtin_amdgcn_exp2f((m - x) * kLog2e) + 1.f;  // m = -inf gives l*0 + 1
      m = x;
    } else if (x > kNegInf) {
      l += __builtin_amdgcn_exp2f((x - m) * kLog2e);
    }
  }
  red_m[tid] = m;
  red_l[tid] = l;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      const float m1 = red_m[tid], m2 = red_m[tid + w];
      const float l1 = red_l[tid], l2 = red_l[tid + w];
      const float mm = fmaxf(m1, m2);
      float ll = 0.f;
      if (mm > kNegInf) {
        ll = (m1 > kNegInf ? l1 * __builtin_amdgcn_exp2f((m1 - mm) * kLog2e) : 0.f) +
             (m2 > kNegInf ? l2 * __builtin_amdgcn_exp2f((m2 - mm) * kLog2e) : 0.f);
      }
      red_m[tid] = mm;
      red_l[tid] = ll;
    }
    __syncthreads();
  }
  const float M = red_m[0];
  const float Lsum = red_l[0];
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  for (int j = tid; j < ld; j += 256) {
    const float x = s[j];
    const float pv = (x > kNegInf) ? __builtin_amdgcn_exp2f((x - M) * kLog2e) * inv : 0.f;
    pr[j] = __builtin_bit_cast(unsigned short, (__bf16)pv);
  }
  if (tid == 0) lse[row] = Lsum > 0.f ? M + __builtin_amdgcn_logf(Lsum) * kLn2 : kNegInf;
}

// ---- launch 3: O = P V --------------------------------------------------------
// One workgroup = 4 waves = 128 rows of O; each wave 32 rows x D.  V tiles of 64
// keys are transposed into LDS so that the B operand (8 consecutive keys of one
// dimension) is a 16-byte read; P rows are read directly from global memory.
template <int D>
__global__ __launch_bounds__(256) void pv_kernel(FwdArgs p, int ld, const unsigned short* P) {
  constexpr int BC = 64;
  constexpr int VSTR = BC + 8;
  __shared__ __attribute__((aligned(16))) unsigned short Vt[D * VSTR];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, lg = lane >> 5;
  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * 128 + 32 * wave;
  const unsigned short* vp = (const unsigned short*)p.v + (size_t)bh * p.Nk * D;
  const unsigned short* ph = P + (size_t)bh * p.Nq * ld;
  unsigned short* op = (unsigned short*)p.o + (size_t)bh * p.Nq * D;
  // V rows past the sequence's key length are never read: their probabilities are 0,
  // but a NaN or Inf there would still turn 0 * x into NaN in the product
  const int L = clamp_len(p.kv_lens, bh / p.H, p.Nk);
  const int j_end = (L + BC - 1) / BC * BC;

  f32x16 acc[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) acc[d] = (f32x16){};
  const int qi = i0 + lq;

  for (int j0 = 0; j0 < j_end; j0 += BC) {
    __syncthreads();
    for (int u = tid; u < (BC / 4) * (D / 8); u += 256) {
      const int kg = u % (BC / 4), dg = u / (BC / 4);
      u32x4 vr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = j0 + 4 * kg + r;
        vr[r] = key < L ? *(const u32x4*)(vp + (size_t)key * D + 8 * dg) : (u32x4){0, 0, 0, 0};
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1, sh = (e & 1) * 16;
        u32x2 pk = {((vr[0][w] >> sh) & 0xFFFFu) | (((vr[1][w] >> sh) & 0xFFFFu) << 16),
                    ((vr[2][w] >> sh) & 0xFFFFu) | (((vr[3][w] >> sh) & 0xFFFFu) << 16)};
        *(u32x2*)(Vt + (8 * dg + e) * VSTR + 4 * kg) = pk;
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < BC / 16; ++s) {
      bf16x8 a = {};
      if (qi < p.Nq) a = *(const bf16x8*)(ph + (size_t)qi * ld + j0 + 16 * s + 8 * lg);
#pragma unroll
      for (int d = 0; d < D / 32; ++d) {
        const bf16x8 bb = *(const bf16x8*)(Vt + (32 * d + lq) * VSTR + 16 * s + 8 * lg);
        acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc[d], 0, 0, 0);
      }
    }
  }
  // accumulator register r of lane l: row 8*(r/4) + 4*(l/32) + r%4, column (dim) l%32
#pragma unroll
  for (int d = 0; d < D / 32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + 8 * (r >> 2) + 4 * lg + (r & 3);
      if (i < p.Nq)
        op[(size_t)i * D + 32 * d + lq] = __builtin_bit_cast(unsigned short, (__bf16)acc[d][r]);
    }
}

}  // namespace

bool materialized_layout(int B, int H, int Nq, int Nk, MatLayout* out) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return false;
  const size_t ld = ((size_t)Nk + 63) / 64 * 64;
  size_t rows = 0, elems = 0;
  if (__builtin_mul_overflow((size_t)B * (size_t)H, (size_t)Nq, &rows)) return false;
  if (__builtin_mul_overflow(rows, ld, &elems)) return false;
  if (elems > ((size_t)1 << 56)) return false;
  out->ld = (int)ld;
  out->s_bytes = elems * 4;
  out->p_offset = (out->s_bytes + 255) / 256 * 256;
  out->total = out->p_offset + elems * 2;
  return true;
}

int launch_attn_materialized(const FwdArgs& a, int D, float scale, void* workspace,
                             const MatLayout& lay, hipStream_t stream) {
  const int BH = a.B * a.H;
  if (BH > 65535) return -8;
  float* S = (float*)workspace;
  unsigned short* P = (unsigned short*)((char*)workspace + lay.p_offset);
  const long long rows = (long long)BH * a.Nq;
  if (rows > 0x7fffffffLL) return -8;
  const int gy1 = (a.Nq + 63) / 64;
  const int gx1 = lay.ld / 64;
  if (gy1 > 65535) return -8;
  dim3 g1(gx1, gy1, BH), g3((a.Nq + 127) / 128, BH);
  if (D == 128) {
    qk_scores_kernel<128><<<g1, 256, 0, stream>>>(a, scale, lay.ld, S);
  } else {
    qk_scores_kernel<64><<<g1, 256, 0, stream>>>(a, scale, lay.ld, S);
  }
  if (hipGetLastError() != hipSuccess) return -7;
  softmax_rows_kernel<<<dim3((unsigned)rows), 256, 0, stream>>>(S, P, a.lse, lay.ld);
  if (hipGetLastError() != hipSuccess) return -7;
  if (D == 128) {
    pv_kernel<128><<<g3, 256, 0, stream>>>(a, lay.ld, P);
  } else {
    pv_kernel<64><<<g3, 256, 0, stream>>>(a, lay.ld, P);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int launch_pv(const FwdArgs& a, int D, int ld, const unsigned short* P, hipStream_t stream) {
  const int BH = a.B * a.H;
  if (BH > 65535) return -8;
  const dim3 g3((a.Nq + 127) / 128, BH);
  if (D == 128)
    pv_kernel<128><<<g3, 256, 0, stream>>>(a, ld, P);
  else
    pv_kernel<64><<<g3, 256, 0, stream>>>(a, ld, P);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace attn89
