// attn_bf16_tiles.hpp -- register and LDS layout helpers shared by the two bf16
// forward kernels (attn_fwd_bf16_pp.hip: 8-wave ping-pong workgroups of 256 rows;
// attn_fwd_bf16_4w.hip: 4-wave workgroups of 128 rows, two per CU).
//
// Both kernels compute the TRANSPOSED scores S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16: A = K (rows = keys, from LDS), B = Q^T (columns =
// queries, in VGPRs for the whole key loop).  Lane l then holds query l%32 and 16
// keys, so a row maximum is an in-lane max plus one exchange with lane l^32, the row
// sum stays per lane until the epilogue, and the per-query rescale is a per-lane
// scalar.  The output is accumulated transposed, O^T = V^T P^T, with P taken straight
// from the score registers as the B operand.  For that, accumulator row i holds key
// swap_bits23(i) (bits 2 and 3 exchanged), so register r of lane l holds key
// 16*(r/8) + 8*(l/32) + r%8 of its 32-key block: the 8 keys a lane contributes to one
// P.V step are consecutive, and so is the matching V^T operand (one dimension, 8
// consecutive keys).
//
// K and V tiles are stored row-major in LDS.  K fragments are single 16-byte reads; the
// V^T operand is gathered from the row-major V tile by two transposing
// ds_read_b64_tr_b16 (lds_tr16).  In both layouts the 16-byte chunks of a row are
// XOR-swizzled with a function of the row, so every fragment read is bank-conflict free
// (the lanes the LDS serves together touch each bank once).
//
// A transposing read is issued by the compiler only after every outstanding load of
// the wave has landed when it cannot tell the read's LDS object from that of a pending
// LDS DMA; the kernels therefore keep each V buffer in a __shared__ array of its own.
#pragma once

#include "common.hpp"

namespace attn89 {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

template <typename T>
__device__ __forceinline__ T lds_load(const lds_u8* base, unsigned off) {
  return *(const __attribute__((address_space(3))) T*)(base + off);
}

// How far (log2 units) the row maximum may rise above the exponent reference before
// the accumulators are corrected.  Online correction, lazily: the exponent reference
// of a row moves to the new row maximum only when the maximum exceeds it by more than
// this (the kernels compare the raw maximum with (reference + this) / (scale log2 e));
// until then exponentials are taken against the older reference and stay at most
// 2^kRescaleSlack, up to the rounding of that comparison.  Numerator and normaliser
// always share one reference, so a / l
// is the same; when the reference moves both are multiplied by
// alpha = exp2(m_old - m_new), the correction of the recurrence.
constexpr float kRescaleSlack = 8.0f;
// 2^(kRescaleSlack - 1): an exponential taken against a reference that has to move is
// above this.  A lane whose exponentials of a tile sum to no more than this has none
// that large, so a kernel may skip the row maxima of that tile.
constexpr float kMoveSum = 128.0f;

// K chunk swizzle: the 16 lanes served together read one chunk column of 16
// consecutive rows; a 128-dimension row spans all 64 banks, a 64-dimension row half.
// Adding 32 to the row leaves it unchanged (so both 32-key blocks share offsets).
template <int D>
__device__ __forceinline__ int kswz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}

// v_permlane32_swap exchanges the upper half-wave of one operand with the lower
// half-wave of the other; with both operands = x, the two results of every lane are
// x[l] and x[l ^ 32] (in some order), so their max / sum is the two-lane reduction.
__device__ __forceinline__ float max_with_partner(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // the inputs are scores or -inf, never NaN: a plain v_max_f32 (fmaxf would first
  // quiet both operands, two more instructions)
  float m;
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
  return m;
}

__device__ __forceinline__ float sum_with_partner(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Swizzle of the 16-byte chunks of a row-major V tile: row bits 0-1
// select the 64-byte window, so a transposing read that gathers four consecutive keys
// touches four windows; it does not change when the row moves by a multiple of 4.
template <int D>
__device__ __forceinline__ int vswz(int row) {
  return D == 128 ? 4 * (row & 3) : 2 * (row & 3);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: 8 bytes (four 16-bit elements) per lane, transposed across each
// group of 16 lanes: lane 16g + 4a + j receives, as its element m, element j of the
// four at the address given by lane 16g + a + 4m (measured on gfx950 with a probe that
// reads back tagged LDS elements)
__device__ __forceinline__ i16x4 lds_tr16(const lds_u8* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<lds_u8*>(p)));
}

__device__ __forceinline__ bf16x8 join_tr16(i16x4 lo, i16x4 hi) {
  const i16x4 v[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ int swap_bits23(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

}  // namespace attn89
