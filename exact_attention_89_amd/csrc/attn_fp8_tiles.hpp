// attn_fp8_tiles.hpp -- layout and arithmetic helpers shared by the two FP8 forward
// kernels (attn_fwd_fp8.hip: 4-wave workgroups of 128 rows, two per CU;
// attn_fwd_fp8_pp.hip: 8-wave ping-pong workgroups of 256 rows).
//
// Both kernels run S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x64_f8f6f4 with
// E4M3 operands.  Lane l feeds row / column l%32 of an operand and 32 consecutive
// bytes (half l/32) of the 64-deep reduction; A and B use the same byte order, so the
// hardware's order inside the reduction cancels.  The score accumulator leaves
// register r of lane l with key 8*(r/4) + 4*(l/32) + r%4 of its 32-key block, so the
// 32 probabilities of a lane over a 64-key tile (two blocks) are one B operand of
// P.V: byte 16*kb + r of half h is key 32*kb + 8*(r/4) + 4*h + r%4.  V^T tiles store
// each dimension's 64 keys in that order (position 32*h + 16*kb + 4*(r/4) + r%4).
#pragma once

#include "attn_bf16_tiles.hpp"

namespace attn89 {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// p' = 2^kPShift * exp2(s*c - m) enters P.V as E4M3: the shift keeps p' in E4M3's
// normal range (relative rounding error <= 2^-4) down to p = 2^-12, and with the
// exponent reference allowed to lag the row maximum by at most kSlack8 (log2 units),
// p' <= 2^(kPShift + kSlack8) = 256 < 448, the largest E4M3 value.
constexpr float kPShift = 6.0f;
constexpr float kSlack8 = 2.0f;

// K chunk swizzle (16-byte chunks): the 16 lanes the LDS serves together read one
// chunk column of 16 consecutive rows; with 128-byte rows two rows span the banks,
// with 64-byte rows four.  Adding 32 to the row leaves it unchanged.
template <int D>
__device__ __forceinline__ int kswz8(int row) {
  return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}
// V^T rows are 64 bytes (4 chunks): four rows span the banks.
__device__ __forceinline__ int vtswz8(int d) { return (d >> 2) & 3; }

typedef int i32x2 __attribute__((ext_vector_type(2)));

// ds_read_b64_tr_b8: 8 bytes per lane, transposed across each group of 16 lanes: lane
// 16g + 8h + j receives, as its byte m, byte j of the 8 bytes at the address given by
// lane 16g + h + 2m (measured on gfx950 with a probe that reads back tagged LDS bytes)
__device__ __forceinline__ i32x2 lds_tr8(const lds_u8* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(const_cast<lds_u8*>(p)));
}

__device__ __forceinline__ i32x8 join_tr8(i32x2 a, i32x2 b, i32x2 c, i32x2 d) {
  return (i32x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ i32x8 join32(u32x4 lo, u32x4 hi) {
  return (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // formats 0/0: both operands E4M3; no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// the 8-byte load of 8 consecutive dimensions
__device__ __forceinline__ u32x2 buffer_load8_so(__amdgpu_buffer_rsrc_t r, unsigned voff,
                                                 int soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// 4 x 4 byte transpose: w_k holds byte x of key k for x = 0..3 (4 dimensions); result
// x holds dimension x of keys 0..3.
__device__ __forceinline__ u32x4 transpose4x4_bytes(unsigned w0, unsigned w1, unsigned w2,
                                                    unsigned w3) {
  const unsigned lo01 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
  const unsigned hi01 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
  const unsigned lo23 = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
  const unsigned hi23 = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
  return (u32x4){__builtin_amdgcn_perm(lo23, lo01, 0x05040100u),
                 __builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
                 __builtin_amdgcn_perm(hi23, hi01, 0x05040100u),
                 __builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};
}

// four weights p' = exp2(s*c - m_sh) (m_sh = reference - kPShift) packed to E4M3 with
// round-to-nearest-even, bytes 0..3 = s0..s3; their fp32 sum is added to lsum
__device__ __forceinline__ int exp2_pack_e4m3(float s0, float s1, float s2, float s3, float c,
                                              float m_sh, float& lsum) {
  const float x0 = __builtin_fmaf(s0, c, -m_sh);
  const float e0 = __builtin_amdgcn_exp2f(x0);
  const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1, c, -m_sh));
  const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s2, c, -m_sh));
  const float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s3, c, -m_sh));
  lsum += (e0 + e1) + (e2 + e3);
  // The first conversion writes bytes 0-1 and keeps bytes 2-3 of its third operand,
  // which the second conversion overwrites: any dead register serves (here x0), so
  // the compiler needs no zeroed register for it.
  const int word = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, __float_as_int(x0), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, word, true);
}

}  // namespace attn89
