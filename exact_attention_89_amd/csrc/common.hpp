// common.hpp -- types and small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn89 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Arguments of the fused forward kernels (device pointers, sizes in elements).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* kv_lens;  // [B] or nullptr
  int B, H, Nq, Nk;
  // Scores enter the exponent as s * c_exp.  When scale > 0, c_exp = scale*log2(e)
  // and the raw dot products are used directly; otherwise the dot products are first
  // multiplied by c_pre = scale*log2(e) and c_exp = 1 (so that -inf masking stays
  // correct for scale <= 0).
  float c_exp;
  float c_pre;
  int pre_scale;  // 1 when c_pre must be applied
  int causal;
  // Split keys (attn_fwd_splitkv only): workgroup split s covers key tiles
  // [s * kv_chunk, (s + 1) * kv_chunk) / 64 and writes its normalised partial output
  // (fp32, [n_splits][B][H][Nq][D]) and partial LSE ([n_splits][B][H][Nq]).
  int n_splits;
  int kv_chunk;   // keys per split, a multiple of 64
  float* o_part;
  float* lse_part;
  // Packed variable-length sequences (attn_fwd_varlen only): sequence b owns tokens
  // [cu_q[b], cu_q[b+1]) of q / o and [cu_k[b], cu_k[b+1]) of k / v; Nq, Nk hold the
  // longest lengths.
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;
};

__device__ __forceinline__ int clamp_len(const int32_t* kv_lens, int b, int nk) {
  if (kv_lens == nullptr) return nk;
  int n = kv_lens[b];
  return n < 0 ? 0 : (n > nk ? nk : n);
}

// Tokens [cu[b], cu[b+1]) of a packed batch: both ends clamped into [0, total] (the
// end not below the start) and the length to at most max_len, so that any offsets
// the caller passes stay inside the tensors the host checks were made for.
struct SeqSpan {
  int start;
  int len;
};
__device__ __forceinline__ SeqSpan seq_span(const int32_t* cu, int b, int total, int max_len) {
  int s = cu[b], e = cu[b + 1];
  s = s < 0 ? 0 : (s > total ? total : s);
  e = e < s ? s : (e > total ? total : e);
  return {s, min(e - s, max_len)};
}

// round-to-nearest-even float -> bf16 bits, two at a time: one v_cvt_pk_bf16_f32
__device__ __forceinline__ unsigned int pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(v, bf16x2));
}

// Buffer resource over [base, base + nbytes): loads at offsets >= nbytes return 0
// (raw buffer addressing, range checked by the hardware), so tails need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// 16 bytes at byte offset voff + soff (soff wave-uniform, in a scalar register)
__device__ __forceinline__ u32x4 buffer_load16_so(__amdgpu_buffer_rsrc_t r, unsigned voff,
                                                  int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Global -> LDS without registers: lane i's 16 bytes from byte offset voff + soff
// land at LDS address lds + 16*i (lds wave-uniform).
__device__ __forceinline__ void buffer_load16_to_lds(__amdgpu_buffer_rsrc_t r,
                                                     __attribute__((address_space(3))) void* lds,
                                                     unsigned voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_float(unsigned short h) {
  return __uint_as_float(((unsigned int)h) << 16);
}

}  // namespace attn89
