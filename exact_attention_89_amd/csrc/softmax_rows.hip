// softmax_rows.hip -- row softmax for gfx950: a fused kernel and the unfused
// four-pass baseline (include/softmax_rows.h).
//
// y_j = exp(x_j - m) / sum_k exp(x_k - m), m = max_k x_k, for every row (page "Kernel
// Fusion and the Memory Wall", section "Softmax needs a global row statistic").  The
// operation is bound by device memory: per element it needs a few vector
// instructions against 8 bytes of traffic at best (one fp32 read, one fp32 write).
// What the two paths differ in is how often a row crosses the memory boundary.
//
// Fused.  One workgroup (256 threads) per row.  Up to 16384 entries the row stays in
// registers (VPT values per thread, loaded in 16-byte vectors when the row allows it)
// from the load through the block maximum, the exponentials, the block sum and the
// division: one read and one write.  Longer rows take two reads: an online pass keeps
// a running (maximum, sum) per thread, rescaling the sum by exp(m_old - m_new) when
// the maximum rises, and a second pass writes exp(x - m) / sum.
//
// Unfused.  Four launches in the page's order: row maxima; exponentials written to y;
// row sums of y; y divided in place.  Four reads and two writes per row.
//
// Masking: -inf entries give exp(-inf - m) = 0.  A row of only -inf entries has
// maximum -inf; its exponent reference is taken as 0 (never -inf - (-inf) = NaN) and
// its zero sum gives an all-zero output.

#include <math.h>

#include "../../include/softmax_rows.h"
#include "common.hpp"

namespace attn89 {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxResident = 16384;   // entries per row kept in registers

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// Stores past the end of the resource are dropped.  They are non-temporal (cache
// policy bit 1, `nt`): every output element is written once and read by nobody in
// the same launch, and streaming the writes past the caches instead of allocating
// lines for them moved 8192 x 8192 from 99 to 77 us (1024 x 65536: 153 to 115 us).
// Loads keep the default policy (non-temporal loads were slower).
constexpr int kStoreNT = 2;
__device__ __forceinline__ void store_f32(float v, __amdgpu_buffer_rsrc_t r, unsigned off) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, off, 0, kStoreNT);
}
__device__ __forceinline__ void store_f32x4(f32x4 v, __amdgpu_buffer_rsrc_t r, unsigned off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kStoreNT);
}

// VEC consecutive floats of a row from element index i (i % VEC == 0); entries at or
// past `cols` read as -inf
template <int VEC>
__device__ __forceinline__ void load_vec(__amdgpu_buffer_rsrc_t r, int i, int cols, float* out) {
  if (VEC == 4) {
    const f32x4 v = __builtin_bit_cast(f32x4, buffer_load16(r, (unsigned)i * 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = (i + e < cols) ? v[e] : kNegInf;
  } else {
    out[0] = (i < cols) ? load_f32(r, (unsigned)i * 4) : kNegInf;
  }
}

template <int VEC>
__device__ __forceinline__ void store_vec(__amdgpu_buffer_rsrc_t r, int i, const float* v) {
  if (VEC == 4)
    store_f32x4((f32x4){v[0], v[1], v[2], v[3]}, r, (unsigned)i * 4);
  else
    store_f32(v[0], r, (unsigned)i * 4);
}

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

// block-wide max / sum of one value per thread (4 waves); every thread gets the result
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float exp_from(float x, float m_use) {
  return __builtin_amdgcn_exp2f((x - m_use) * kLog2e);
}

// ---- fused: the row in registers ----
template <int VPT, int VEC>
__global__ __launch_bounds__(kThreads) void softmax_resident_kernel(const float* x, float* y,
                                                                    int cols) {
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + row * cols, (unsigned)cols * 4);
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(y + row * cols, (unsigned)cols * 4);
  constexpr int STEPS = VPT / VEC;
  float v[VPT];
#pragma unroll
  for (int s = 0; s < STEPS; ++s)
    load_vec<VEC>(xr, (s * kThreads + (int)threadIdx.x) * VEC, cols, &v[s * VEC]);
  float m = kNegInf;
#pragma unroll
  for (int k = 0; k < VPT; ++k) m = fmaxf(m, v[k]);
  m = block_max(m, red);
  const float m_use = (m == kNegInf) ? 0.f : m;
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    v[k] = exp_from(v[k], m_use);
    sum += v[k];
  }
  sum = block_sum(sum, red);
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) v[k] *= inv;
#pragma unroll
  for (int s = 0; s < STEPS; ++s)
    store_vec<VEC>(yr, (s * kThreads + (int)threadIdx.x) * VEC, &v[s * VEC]);
}

// ---- fused: long rows, online pass then writing pass ----
template <int VEC>
__global__ __launch_bounds__(kThreads) void softmax_stream_kernel(const float* x, float* y,
                                                                  int cols) {
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + row * cols, (unsigned)cols * 4);
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(y + row * cols, (unsigned)cols * 4);
  constexpr int U = 4;                       // vectors per step
  constexpr int STEP = kThreads * VEC * U;
  float m = kNegInf, l = 0.f;
  for (int c0 = 0; c0 < cols; c0 += STEP) {
    float v[U * VEC];
#pragma unroll
    for (int u = 0; u < U; ++u)
      load_vec<VEC>(xr, c0 + (u * kThreads + (int)threadIdx.x) * VEC, cols, &v[u * VEC]);
    float cm = kNegInf;
#pragma unroll
    for (int k = 0; k < U * VEC; ++k) cm = fmaxf(cm, v[k]);
    const float m_new = fmaxf(m, cm);
    const float mu = (m_new == kNegInf) ? 0.f : m_new;
    // the online correction: the old sum was taken against m (exp(-inf) = 0 when
    // nothing valid has been seen, and l is 0 then anyway)
    float s = l * exp_from(m, mu);
#pragma unroll
    for (int k = 0; k < U * VEC; ++k) s += exp_from(v[k], mu);
    l = s;
    m = m_new;
  }
  const float M = block_max(m, red);
  const float mu = (M == kNegInf) ? 0.f : M;
  const float L = block_sum(l * exp_from(m, mu), red);
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  for (int c0 = 0; c0 < cols; c0 += STEP) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = c0 + (u * kThreads + (int)threadIdx.x) * VEC;
      float v[VEC];
      load_vec<VEC>(xr, i, cols, v);
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = exp_from(v[e], mu) * inv;
      store_vec<VEC>(yr, i, v);
    }
  }
}

// ---- unfused: four launches ----
template <int VEC>
__global__ __launch_bounds__(kThreads) void row_max_kernel(const float* x, float* mx, int cols) {
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + row * cols, (unsigned)cols * 4);
  float m = kNegInf;
  for (int i = (int)threadIdx.x * VEC; i < cols; i += kThreads * VEC) {
    float v[VEC];
    load_vec<VEC>(xr, i, cols, v);
#pragma unroll
    for (int e = 0; e < VEC; ++e) m = fmaxf(m, v[e]);
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) mx[row] = m;
}

template <int VEC>
__global__ __launch_bounds__(kThreads) void exp_write_kernel(const float* x, const float* mx,
                                                             float* y, int cols) {
  const size_t row = blockIdx.x;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + row * cols, (unsigned)cols * 4);
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(y + row * cols, (unsigned)cols * 4);
  const float m = mx[row];
  const float m_use = (m == kNegInf) ? 0.f : m;
  for (int i = (int)threadIdx.x * VEC; i < cols; i += kThreads * VEC) {
    float v[VEC];
    load_vec<VEC>(xr, i, cols, v);
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] = exp_from(v[e], m_use);
    store_vec<VEC>(yr, i, v);
  }
}

template <int VEC>
__global__ __launch_bounds__(kThreads) void row_sum_kernel(const float* y, float* sm, int cols) {
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(y + row * cols, (unsigned)cols * 4);
  float s = 0.f;
  for (int i = (int)threadIdx.x * VEC; i < cols; i += kThreads * VEC) {
    float v[VEC];
    load_vec<VEC>(yr, i, cols, v);   // past the end: -inf, excluded below
#pragma unroll
    for (int e = 0; e < VEC; ++e) s += (i + e < cols) ? v[e] : 0.f;
  }
  s = block_sum(s, red);
  if (threadIdx.x == 0) sm[row] = s;
}

template <int VEC>
__global__ __launch_bounds__(kThreads) void normalize_kernel(float* y, const float* sm, int cols) {
  const size_t row = blockIdx.x;
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(y + row * cols, (unsigned)cols * 4);
  const float s = sm[row];
  const float inv = s > 0.f ? 1.0f / s : 0.f;
  for (int i = (int)threadIdx.x * VEC; i < cols; i += kThreads * VEC) {
    float v[VEC];
    load_vec<VEC>(yr, i, cols, v);
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] *= inv;
    store_vec<VEC>(yr, i, v);
  }
}

template <int VEC>
int launch_fused(const float* x, float* y, int rows, int cols, hipStream_t st) {
  const dim3 g((unsigned)rows), b(kThreads);
  if (cols <= 1024 * 1)
    softmax_resident_kernel<4, VEC><<<g, b, 0, st>>>(x, y, cols);
  else if (cols <= 2048)
    softmax_resident_kernel<8, VEC><<<g, b, 0, st>>>(x, y, cols);
  else if (cols <= 4096)
    softmax_resident_kernel<16, VEC><<<g, b, 0, st>>>(x, y, cols);
  else if (cols <= 8192)
    softmax_resident_kernel<32, VEC><<<g, b, 0, st>>>(x, y, cols);
  else if (cols <= kMaxResident)
    softmax_resident_kernel<64, VEC><<<g, b, 0, st>>>(x, y, cols);
  else
    softmax_stream_kernel<VEC><<<g, b, 0, st>>>(x, y, cols);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

template <int VEC>
int launch_unfused(const float* x, float* y, int rows, int cols, float* mx, float* sm,
                   hipStream_t st) {
  const dim3 g((unsigned)rows), b(kThreads);
  row_max_kernel<VEC><<<g, b, 0, st>>>(x, mx, cols);
  exp_write_kernel<VEC><<<g, b, 0, st>>>(x, mx, y, cols);
  row_sum_kernel<VEC><<<g, b, 0, st>>>(y, sm, cols);
  normalize_kernel<VEC><<<g, b, 0, st>>>(y, sm, cols);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check(const float* x, const float* y, int rows, int cols) {
  if (!x || !y) return ATTN_ERR_NULL;
  if (rows < 1 || cols < 1) return ATTN_ERR_SHAPE;
  if ((size_t)cols * 4 >= ((size_t)1 << 31)) return ATTN_ERR_TOO_LARGE;
  if (!aligned(x, 4) || !aligned(y, 4)) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

// 16-byte vectors when every row starts 16-byte aligned
bool use_vec4(const float* x, const float* y, int cols) {
  return cols % 4 == 0 && aligned(x, 16) && aligned(y, 16);
}

size_t workspace_bytes(int rows) {
  const size_t half = (((size_t)rows * 4) + 255) / 256 * 256;
  return 2 * half;
}

}  // namespace
}  // namespace attn89

extern "C" {

int softmax_rows_f32(const float* x, float* y, int rows, int cols, void* stream) {
  const int st = attn89::check(x, y, rows, cols);
  if (st != ATTN_OK) return st;
  if (attn89::use_vec4(x, y, cols))
    return attn89::launch_fused<4>(x, y, rows, cols, (hipStream_t)stream);
  return attn89::launch_fused<1>(x, y, rows, cols, (hipStream_t)stream);
}

size_t softmax_rows_unfused_workspace_bytes(int rows) {
  return rows < 1 ? 0 : attn89::workspace_bytes(rows);
}

int softmax_rows_unfused_f32(const float* x, float* y, int rows, int cols, void* workspace,
                             size_t workspace_bytes, void* stream) {
  const int st = attn89::check(x, y, rows, cols);
  if (st != ATTN_OK) return st;
  if (!workspace || workspace_bytes < attn89::workspace_bytes(rows) ||
      ((uintptr_t)workspace % 256) != 0)
    return ATTN_ERR_WORKSPACE;
  float* mx = (float*)workspace;
  float* sm = (float*)((char*)workspace + attn89::workspace_bytes(rows) / 2);
  if (attn89::use_vec4(x, y, cols))
    return attn89::launch_unfused<4>(x, y, rows, cols, mx, sm, (hipStream_t)stream);
  return attn89::launch_unfused<1>(x, y, rows, cols, mx, sm, (hipStream_t)stream);
}

}  // extern "C"
