// attn_splitkv.hip -- split keys: the key range of every (batch, head, query block)
// is cut into n_splits chunks that separate workgroups process in parallel, then one
// merge launch combines the partial results.
//
// For few queries and many keys (decoding against a long or ragged KV cache) one
// workgroup per (batch, head) leaves most of the GPU idle; splitting the keys
// multiplies the workgroups.  Split s (4-wave kernel, SPLIT instantiation) computes
// the attention of its queries over its key range only, normalised by its own sum:
// O_s and LSE_s = log sum over its keys of exp(score).  The rows of the full
// softmax follow from the same rescaling the online recurrence uses (page "Attention
// softmax fusion", section "The tile loop": the sums kept so far are scaled by
// exp(m_old - m_new) when a new part raises the maximum), applied to whole ranges:
//
//   LSE = log sum_s exp(LSE_s)            (computed against the largest LSE_s)
//   O   = sum_s exp(LSE_s - LSE) O_s
//
// A range without a valid key has LSE_s = -inf and weight 0; a row without any valid
// key has every LSE_s = -inf and gets O = 0, LSE = -inf, the convention of attn_fwd.

#include "common.hpp"
#include "launch.hpp"

namespace attn89 {
namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// one wave per (batch, head, query) row, four rows per workgroup; the split weights
// are computed once per row (lanes over splits) and kept in LDS, then every lane
// accumulates its output dimensions over the splits with several loads in flight
constexpr int kMaxSplitsLds = 256;

template <int D>
__global__ __launch_bounds__(256) void splitkv_merge_kernel(FwdArgs p) {
  __shared__ float wts[4][kMaxSplitsLds];
  const long long rows = (long long)p.B * p.H * p.Nq;
  const int w = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * 4 + w;
  const int lane = threadIdx.x & 63;
  const int S = p.n_splits;
  const bool live = row < rows;
  float mx = kNegInf;
  if (live)
    for (int s = lane; s < S; s += 64) mx = fmaxf(mx, p.lse_part[(size_t)s * rows + row]);
  mx = wave_max(mx);
  const float ref = (mx == kNegInf) ? 0.f : mx;
  float den = 0.f;
  if (live)
    for (int s = lane; s < S; s += 64) {
      const float e = expf(p.lse_part[(size_t)s * rows + row] - ref);   // 0 for empty ranges
      wts[w][s] = e;
      den += e;
    }
  den = wave_sum(den);
  __syncthreads();
  if (!live) return;
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  constexpr int E = D / 64;          // output dimensions per lane
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll 8
  for (int s = 0; s < S; ++s) {
    const float* orow = p.o_part + ((size_t)s * rows + row) * D + lane * E;
    const float ws = wts[w][s];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += ws * orow[e];
  }
  unsigned short* o = (unsigned short*)p.o + (size_t)row * D + lane * E;
  if (E == 2) {
    *(unsigned*)o = pack_bf16x2(acc[0] * inv, acc[E - 1] * inv);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const unsigned pk = pack_bf16x2(acc[e] * inv, 0.f);
      o[e] = (unsigned short)(pk & 0xFFFFu);
    }
  }
  if (lane == 0) p.lse[row] = den > 0.f ? ref + logf(den) : kNegInf;
}

}  // namespace

int splitkv_plan(int B, int H, int Nq, int Nk, int requested, int num_cus, int* chunk) {
  const long long tiles = ((long long)Nk + 63) / 64;
  long long splits = requested;
  if (splits <= 0) {
    const long long base = ((long long)Nq + 127) / 128 * B * H;
    const long long target = 2LL * num_cus;          // two 4-wave workgroups per CU
    splits = (target + base - 1) / base;
    if (splits > 64) splits = 64;
  }
  if (splits > 256) splits = 256;   // the merge keeps one weight per split in LDS
  if (splits > tiles) splits = tiles;
  if (splits < 1) splits = 1;
  const long long per = (tiles + splits - 1) / splits;  // tiles per split
  *chunk = (int)(per * 64);
  return (int)((tiles + per - 1) / per);               // splits that cover the keys
}

int launch_attn_splitkv(const FwdArgs& a, int D, hipStream_t stream) {
  int st = launch_attn_fwd_bf16_4w_split(a, D, stream);
  if (st != 0) return st;
  const long long rows = (long long)a.B * a.H * a.Nq;
  const long long blocks = (rows + 3) / 4;
  if (blocks > 0x7fffffffLL) return -8;
  if (D == 128)
    splitkv_merge_kernel<128><<<dim3((unsigned)blocks), 256, 0, stream>>>(a);
  else
    splitkv_merge_kernel<64><<<dim3((unsigned)blocks), 256, 0, stream>>>(a);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace attn89
