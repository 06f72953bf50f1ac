// attn_fwd_f32.hip -- the fused attention forward, float32 in / float32 out.
//
// Same method as the bf16 kernel (one launch, online softmax over key tiles held
// in LDS, deferred normalisation; page "Attention softmax fusion", section "The
// tile loop"; page "Kernel Fusion and the Memory Wall", section "FlashAttention:
// avoid the full score matrix"), with every product in fp32 on the vector ALUs and
// no rounding of P.  It serves float32 callers; the throughput path is bf16.
//
// Work split: one workgroup = 256 threads = 64 query rows; four consecutive lanes
// share a row and each owns the dimensions d = 4*i + part, so the four partial dot
// products are combined with two lane exchanges and every K/V read from LDS is a
// broadcast of 4 consecutive words.  Keys are streamed in tiles of 32.

#include "common.hpp"
#include "launch.hpp"

namespace attn89 {
namespace {

constexpr int F_BR = 64;
constexpr int F_BC = 32;

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(FwdArgs p) {
  constexpr int DP = D / 4;  // dimensions owned by one lane
  __shared__ __attribute__((aligned(16))) float Ks[F_BC * D];
  __shared__ __attribute__((aligned(16))) float Vs[F_BC * D];

  const int tid = threadIdx.x;
  const int part = tid & 3;
  const int BH = p.B * p.H;
  const int n_qb = (p.Nq + F_BR - 1) / F_BR;
  const int qb = n_qb - 1 - (int)blockIdx.x / BH;
  const int bh = (int)blockIdx.x % BH;
  const int b = bh / p.H;

  const float* qp = (const float*)p.q + (size_t)bh * p.Nq * D;
  const float* kp = (const float*)p.k + (size_t)bh * p.Nk * D;
  const float* vp = (const float*)p.v + (size_t)bh * p.Nk * D;
  float* op = (float*)p.o + (size_t)bh * p.Nq * D;

  const int L = clamp_len(p.kv_lens, b, p.Nk);
  const int q0 = qb * F_BR;
  const int row = q0 + (tid >> 2);
  const int q_hi = min(q0 + F_BR, p.Nq);
  const int kv_end = p.causal ? min(L, q_hi) : L;
  const int n_tiles = (kv_end + F_BC - 1) / F_BC;

  float qv[DP], ov[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    qv[i] = row < p.Nq ? qp[(size_t)row * D + 4 * i + part] : 0.f;
    ov[i] = 0.f;
  }
  float m_run = kNegInf, l_run = 0.f;

  for (int t = 0; t < n_tiles; ++t) {
    const int j0 = t * F_BC;
    __syncthreads();  // previous tile fully consumed
    for (int c = tid; c < F_BC * D / 4; c += 256) {
      const int kr = c / (D / 4);
      const int col = (c % (D / 4)) * 4;
      const int key = j0 + kr;
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (key < L) {
        kx = *(const f32x4*)(kp + (size_t)key * D + col);
        vx = *(const f32x4*)(vp + (size_t)key * D + col);
      }
      *(f32x4*)(Ks + kr * D + col) = kx;
      *(f32x4*)(Vs + kr * D + col) = vx;
    }
    __syncthreads();

    float s[F_BC];
#pragma unroll
    for (int j = 0; j < F_BC; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < DP; ++i) acc = __builtin_fmaf(qv[i], Ks[j * D + 4 * i + part], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      if (p.pre_scale) acc *= p.c_pre;
      const int key = j0 + j;
      const bool ok = key < L && (!p.causal || key <= row);
      s[j] = ok ? acc : kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < F_BC; ++j) mx = fmaxf(mx, s[j]);
    const float m_new = fmaxf(m_run, mx * p.c_exp);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;  // guard: no -inf - (-inf)
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < F_BC; ++j) {
      s[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], p.c_exp, -m_use));
      lsum += s[j];
    }
    l_run = alpha * l_run + lsum;
#pragma unroll
    for (int i = 0; i < DP; ++i) {
      float acc = ov[i] * alpha;
#pragma unroll
      for (int j = 0; j < F_BC; ++j) acc = __builtin_fmaf(s[j], Vs[j * D + 4 * i + part], acc);
      ov[i] = acc;
    }
  }

  if (row < p.Nq) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
#pragma unroll
    for (int i = 0; i < DP; ++i) op[(size_t)row * D + 4 * i + part] = ov[i] * inv;
    if (part == 0) {
      p.lse[(size_t)bh * p.Nq + row] =
          l_run > 0.f ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : kNegInf;
    }
  }
}

}  // namespace

int launch_attn_fwd_f32(const FwdArgs& a, int D, hipStream_t stream) {
  const int n_qb = (a.Nq + F_BR - 1) / F_BR;
  const long long grid = (long long)n_qb * a.B * a.H;
  if (grid > 0x7fffffffLL) return -8;
  if (D == 128) {
    attn_fwd_f32_kernel<128><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(a);
  } else {
    attn_fwd_f32_kernel<64><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace attn89
