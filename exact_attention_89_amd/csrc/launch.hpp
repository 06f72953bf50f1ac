// launch.hpp -- host-side launchers of the kernels (internal to the library).
// Each returns 0, or a negative status of include/attn.h.  Arguments are validated
// by the caller (attn_api.hip) before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace attn89 {

// bf16 forward kernels: 8-wave ping-pong workgroups of 256 query rows (D = 128 only)
// and 4-wave workgroups of 128 rows (any supported D); key_groups = 2 gives the latter
// 8 waves that split each row block's key tiles between two groups.
int launch_attn_fwd_bf16_pp(const FwdArgs& a, int D, hipStream_t stream);
int launch_attn_fwd_bf16_4w(const FwdArgs& a, int D, hipStream_t stream, int key_groups = 1);
// 4-wave kernel over one key range per workgroup (FwdArgs n_splits, kv_chunk,
// o_part, lse_part), partial results only
int launch_attn_fwd_bf16_4w_split(const FwdArgs& a, int D, hipStream_t stream);
// 4-wave kernel over packed variable-length sequences (FwdArgs cu_q, cu_k, total_q,
// total_k; Nq, Nk = the longest lengths)
int launch_attn_fwd_bf16_4w_varlen(const FwdArgs& a, int D, hipStream_t stream);

// Split keys: number of splits actually used for a request (<= 0: automatic, aiming
// at two workgroups per CU) and the keys per split (*chunk, a multiple of 64).
int splitkv_plan(int B, int H, int Nq, int Nk, int requested, int num_cus, int* chunk);
// The split kernel, then the merge into o and lse.
int launch_attn_splitkv(const FwdArgs& a, int D, hipStream_t stream);
int launch_attn_fwd_f32(const FwdArgs& a, int D, hipStream_t stream);
// FP8 (E4M3) forward, 4-wave workgroups; c_exp / c_pre carry scale * q_descale *
// k_descale, v_descale multiplies the output.
int launch_attn_fwd_fp8(const FwdArgs& a, int D, float v_descale, hipStream_t stream);
// the same in 8-wave ping-pong workgroups of 256 rows
int launch_attn_fwd_fp8_pp(const FwdArgs& a, int D, float v_descale, hipStream_t stream);

// Workspace layout of the materialised baseline: S (fp32) then P (bf16), both
// [B][H][Nq][ld] with ld = Nk rounded up to a multiple of 64.
struct MatLayout {
  int ld;
  size_t s_bytes;
  size_t p_offset;
  size_t total;
};
bool materialized_layout(int B, int H, int Nq, int Nk, MatLayout* out);
int launch_attn_materialized(const FwdArgs& a, int D, float scale, void* workspace,
                             const MatLayout& lay, hipStream_t stream);

// O = P V for a probability matrix P (bf16, [B][H][Nq][ld], every column < ld
// defined, zeros where masked); the third launch of the materialised baseline.
int launch_pv(const FwdArgs& a, int D, int ld, const unsigned short* P, hipStream_t stream);

// Partial fusion: QK^T and softmax in one launch writing P (bf16) and LSE, then
// launch_pv.  P: [B][H][Nq][ld], ld = Nk rounded up to 64.
int launch_attn_partial(const FwdArgs& a, int D, int ld, unsigned short* P, hipStream_t stream);

}  // namespace attn89
