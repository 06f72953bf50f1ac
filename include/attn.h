/*
 * attn.h -- C ABI of the exact fused attention library for MI355X (gfx950).
 *
 * The operation (page "Kernel Fusion and the Memory Wall", section
 * "FlashAttention: avoid the full score matrix"):
 *
 *     O = softmax(Q K^T * scale + mask) V,   LSE_i = log sum_j exp(s_ij)
 *
 * computed in ONE kernel that keeps the score tile, the row maximum and sum,
 * the exponentials, the online rescale by exp(m_old - m_new) and the P.V
 * contraction on chip (page "Attention softmax fusion", sections "What fused
 * has to mean" and "The tile loop"), so no Nq x Nk score or probability tensor
 * is ever written to device memory.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer on the current HIP device.  The
 *   caller owns and allocates every buffer; the library allocates nothing and
 *   keeps no state between calls (it is reentrant).
 * - Layout: contiguous row-major [B][H][N][D]; q and o use Nq rows, k and v
 *   use Nk rows.  lse is [B][H][Nq] float32.  kv_lens is [B] int32 (device
 *   memory) or NULL.
 * - Mask: key j is valid for query i iff j < kv_len[b] and, when causal != 0,
 *   j <= i (top-left aligned; also when Nq != Nk).  kv_len values outside
 *   [0, Nk] are clamped into it; NULL means kv_len = Nk for every sequence.
 *   kv_lens is read on the device only, never on the host.
 * - A query row with no valid key gets O = 0 and LSE = -inf (never NaN).
 * - LSE is the natural-log log-sum-exp of the scaled, masked scores.
 * - scale is any finite float (typically 1/sqrt(D)).
 * - Calls are stream-ordered: they enqueue work on `stream` (a hipStream_t;
 *   NULL is the null stream) and return before it finishes.  A fault during
 *   execution surfaces at the caller's next synchronisation.
 * - On any error a negative status is returned, nothing is launched and no
 *   output byte is written.
 * - o and lse must not alias q, k, v or each other.
 */
#ifndef EXACT_ATTENTION_89_ATTN_H
#define EXACT_ATTENTION_89_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define ATTN_OK               0
#define ATTN_ERR_NULL        -1  /* a required pointer is NULL                         */
#define ATTN_ERR_SHAPE       -2  /* B, H, Nq or Nk < 1, or a size overflows 64 bits    */
#define ATTN_ERR_UNSUPPORTED -3  /* head dimension D is not 64 or 128                  */
#define ATTN_ERR_ALIGN       -4  /* q, k, v or o not 16-byte aligned, lse/kv_lens not 4 */
#define ATTN_ERR_SCALE       -5  /* scale is NaN or infinite                           */
#define ATTN_ERR_WORKSPACE   -6  /* workspace NULL or smaller than required            */
#define ATTN_ERR_HIP         -7  /* the HIP runtime reported an error at launch        */
#define ATTN_ERR_TOO_LARGE   -8  /* grid would exceed the launch limits                */
#define ATTN_ERR_SCRATCH     -9  /* more scratch than attn_fwd_splitkv_noalloc holds   */

/*
 * attn_fwd -- the fused forward, bfloat16 inputs and output.
 *
 * q [B][H][Nq][D], k and v [B][H][Nk][D]: bfloat16 (raw 16-bit patterns).
 * o [B][H][Nq][D]: bfloat16, written by round-to-nearest-even from the fp32
 * result.  lse [B][H][Nq]: float32.  Products Q.K^T and P.V run on bf16
 * matrix instructions with fp32 accumulation; P is rounded to bf16 before the
 * P.V product, the softmax statistics stay in fp32.
 *
 * The whole computation is one kernel launch.  Tile loop: page "Attention
 * softmax fusion", section "The tile loop"; online correction and deferred
 * normalisation: page "Kernel Fusion and the Memory Wall", section
 * "FlashAttention: avoid the full score matrix"; guard for fully masked
 * tiles: page "Attention softmax fusion", section "Things that break".
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Nq, int Nk, int D, float scale, int causal,
             const int32_t* kv_lens, void* stream);

/*
 * attn_fwd_select_kernel -- which forward kernel attn_fwd (bf16) and attn_fwd_fp8
 * (E4M3) launch.  For each input type the ping-pong and four-wave kernels compute the
 * same function with the same arithmetic (bitwise identical results); they differ
 * only in how work is spread over the GPU:
 *
 *   ATTN_KERNEL_PINGPONG  8-wave workgroups of 256 query rows, two wave groups
 *                         half a key tile apart (one on the matrix cores while
 *                         the other computes its softmax); one workgroup per CU
 *   ATTN_KERNEL_FOURWAVE  4-wave workgroups of 128 query rows, two per CU
 *   ATTN_KERNEL_KEYGROUPS (bf16 only) 8-wave workgroups of 128 query rows whose two
 *                         4-wave groups take alternate key tiles of the same rows
 *                         and combine their partial results at the end (page
 *                         "Attention softmax fusion", section "The tile loop": the
 *                         rescaling by exp(m_old - m_new) joins any two parts);
 *                         half the sequential key loop per workgroup, for grids
 *                         too small to fill the GPU.  Same function and tolerance,
 *                         a different summation order (not bitwise equal to the
 *                         others); attn_fwd_fp8 treats it as FOURWAVE
 *   ATTN_KERNEL_AUTO      (default) attn_fwd: ping-pong when D = 128, Nq >= 256
 *                         and its grid, ceil(Nq/256)*B*H workgroups, covers every
 *                         compute unit; otherwise key groups when ceil(Nq/128)*B*H
 *                         is at most the number of compute units (one four-wave
 *                         workgroup per CU would leave half of each CU idle and
 *                         the longest key loop alone would set the time); otherwise
 *                         four-wave.  attn_fwd_fp8: four-wave (the faster one for
 *                         FP8 at every measured shape)
 *
 * The setting is process-wide and not synchronised: change it only while no
 * other thread calls attn_fwd.  Returns the previous setting, or
 * ATTN_ERR_UNSUPPORTED (setting unchanged) for any other value of `which`.
 */
#define ATTN_KERNEL_AUTO      0
#define ATTN_KERNEL_PINGPONG  1
#define ATTN_KERNEL_FOURWAVE  2
#define ATTN_KERNEL_KEYGROUPS 3
int attn_fwd_select_kernel(int which);

/*
 * attn_fwd_varlen -- the fused forward over a packed batch of variable-length
 * sequences (page "Fused Multi-Head Attention", section on how fused attention
 * combines with other inference techniques: the ragged tensors of continuous
 * batching), bfloat16 in / out.
 *
 * q, o [total_q][H][D], k, v [total_k][H][D]: bfloat16, token-major, the heads of a
 * token adjacent (rows of one head are H*D elements apart).  Sequence b (0 <= b < B)
 * owns query tokens [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key/value tokens
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]); its queries attend to its own keys only.
 * cu_seqlens_q, cu_seqlens_k: device int32 arrays of B + 1 entries, normally
 * nondecreasing from 0 to total_q / total_k (not read on the host).  The kernel
 * clamps every entry into [0, total], an end below its start to the start, and a
 * length above max_seqlen_q / max_seqlen_k to that maximum; query rows outside the
 * clamped sequences are not written, and rows two clamped sequences share (only
 * possible when the offsets decrease) hold the result of either.  lse [H][total_q]: float32, the LSE of query
 * token t and head h at lse[h * total_q + t].  Causal masking is top-left within
 * each sequence (its key j is visible to its query i iff j <= i); a sequence with no
 * keys gives O = 0 and LSE = -inf.  One launch of the four-wave kernel.
 *
 * Errors as attn_fwd, plus: ATTN_ERR_NULL for a NULL cu_seqlens array,
 * ATTN_ERR_SHAPE for total_q, total_k, max_seqlen_q or max_seqlen_k < 1,
 * ATTN_ERR_TOO_LARGE when (max_seqlen + 256) * H * D * 2 bytes reaches 2^31.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int H,
                    int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int D,
                    float scale, int causal, void* stream);

/*
 * attn_fwd_fp8 -- the fused forward on FP8 inputs (page "Fused Multi-Head
 * Attention", quantization item of the section on how fused attention combines
 * with other inference techniques: FP8 data for the matrix products).
 *
 * q [B][H][Nq][D], k and v [B][H][Nk][D]: OCP E4M3 codes (one byte each: sign,
 * 4-bit exponent with bias 7, 3-bit fraction; 0x7F and 0xFF are NaN and must not
 * occur).  The values they stand for are q_descale * q, k_descale * k and
 * v_descale * v (one float32 factor per tensor, positive and finite, else
 * ATTN_ERR_SCALE).  o [B][H][Nq][D]: bfloat16 (round-to-nearest-even); lse
 * [B][H][Nq]: float32.  Same masks, conventions (fully masked rows: O = 0,
 * LSE = -inf) and errors as attn_fwd; a single kernel launch.
 *
 * Arithmetic: Q.K^T and P.V run on FP8 matrix instructions with fp32
 * accumulation; scores are scaled by fp32(scale * q_descale * k_descale); the
 * softmax statistics stay in fp32; the probabilities are rounded to E4M3 (after
 * a factor 2^6 that keeps them in E4M3's normal range) before P.V, so each
 * weight carries a relative error of at most 2^-4 where p >= 2^-12 times the
 * row maximum's weight; the normaliser sums the unrounded weights.
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Nq, int Nk, int D, float scale, float q_descale,
                 float k_descale, float v_descale, int causal, const int32_t* kv_lens,
                 void* stream);

/*
 * attn_fwd_f32 -- the same fused forward for float32 inputs and output.
 * Same arguments and semantics as attn_fwd, with float32 q, k, v, o.  All
 * arithmetic is fp32 (no rounding of P).
 */
int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                 int B, int H, int Nq, int Nk, int D, float scale, int causal,
                 const int32_t* kv_lens, void* stream);

/*
 * attn_materialized_workspace_bytes -- bytes of workspace attn_materialized
 * needs: the full score matrix S (float32) and the probability matrix P
 * (bfloat16), B*H*Nq*Nk*(4 + 2) bytes plus alignment padding.  Returns 0 when
 * a size is < 1 or the product overflows.
 */
size_t attn_materialized_workspace_bytes(int B, int H, int Nq, int Nk);

/*
 * attn_materialized -- the unfused three-kernel baseline, kept only to show
 * the device-memory traffic that fusion removes (page "Fused Multi-Head
 * Attention", the list of separate launches: score GEMM, softmax kernel,
 * weighted-sum GEMM; page "Attention softmax fusion", section "What fused has
 * to mean").
 *
 *   launch 1  S = scale * Q K^T, masked entries = -inf      -> workspace (fp32)
 *   launch 2  P = softmax(S) row by row, LSE                -> workspace (bf16), lse
 *   launch 3  O = P V                                        -> o
 *
 * Inputs, outputs and mask semantics as attn_fwd (bfloat16).  `workspace` is
 * a caller-owned device buffer of at least
 * attn_materialized_workspace_bytes(B, H, Nq, Nk) bytes, 256-byte aligned; its
 * contents on return are unspecified.
 */
int attn_materialized(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Nq, int Nk, int D, float scale, int causal,
                      const int32_t* kv_lens, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * attn_partial_workspace_bytes -- bytes of workspace attn_partial needs: the
 * probability matrix P (bfloat16), B*H*Nq*ld*2 bytes with ld = Nk rounded up to
 * 64, plus alignment padding.  Returns 0 when a size is < 1 or overflows.
 */
size_t attn_partial_workspace_bytes(int B, int H, int Nq, int Nk);

/*
 * attn_partial -- partial fusion, two launches.  The first kernel fuses Q.K^T
 * with the softmax (a score tile is normalised without leaving the chip) and
 * stores the probabilities P (bfloat16) in the workspace; the second computes
 * O = P V from them (page "Attention softmax fusion", section "What fused has
 * to mean": with only that boundary fused, a score-sized tensor still goes
 * through device memory).  The first kernel visits the
 * key tiles twice (row statistics, then P), so it spends twice the Q.K^T
 * arithmetic of attn_fwd; masked entries and key tiles no query of a block can
 * see are written as zeros, so every column below ld is defined.
 *
 * Inputs, outputs and mask semantics as attn_fwd (bfloat16); same tolerance.
 * `workspace`: caller-owned device buffer of at least
 * attn_partial_workspace_bytes(B, H, Nq, Nk) bytes, 256-byte aligned
 * (ATTN_ERR_WORKSPACE otherwise); on return it holds P.  B*H must be at most
 * 65535 (ATTN_ERR_TOO_LARGE).
 */
int attn_partial(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Nq, int Nk, int D, float scale, int causal,
                 const int32_t* kv_lens, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * attn_fwd_splitkv -- the fused forward (same arguments, semantics and
 * tolerance as attn_fwd, bfloat16) with the keys of every (batch, head, query
 * block) split into ranges that run as separate workgroups, for calls with few
 * queries and many keys (decoding against a KV cache: Nq small, Nk large or
 * kv_lens ragged), where one workgroup per (batch, head) would leave the GPU
 * idle.  Each range writes its normalised partial output O_s (fp32) and
 * LSE_s to the workspace; a merge launch combines them:
 * LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s (the online
 * correction of page "Attention softmax fusion", section "The tile loop",
 * applied to whole key ranges).  Two launches; the split kernel is the 4-wave
 * bf16 kernel restricted to a key range.
 *
 * num_splits: requested number of key ranges (<= 0: automatic, about two
 * workgroups per compute unit); it is clamped to [1, min(256, ceil(Nk / 64))] and the
 * ranges are whole 64-key tiles, so fewer ranges may be used
 * (attn_splitkv_num_splits returns the number).  `workspace`: caller-owned
 * device buffer of at least attn_splitkv_workspace_bytes(B, H, Nq, Nk, D,
 * num_splits) bytes (the same num_splits), 256-byte aligned
 * (ATTN_ERR_WORKSPACE otherwise); its contents on return are unspecified.
 */
int attn_splitkv_num_splits(int B, int H, int Nq, int Nk, int num_splits);
size_t attn_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int D, int num_splits);
int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int Nq, int Nk, int D, float scale, int causal,
                     const int32_t* kv_lens, int num_splits, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * attn_fwd_splitkv_noalloc -- attn_fwd_splitkv without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The partial results live in a fixed scratch array of the library
 * (ATTN_NOALLOC_SCRATCH_BYTES per device, allocated when the library is loaded
 * and held until the process ends); the caller still owns q, k, v, o, lse and
 * kv_lens.  Same arguments (minus workspace), semantics, kernels and results as
 * attn_fwd_splitkv with the same num_splits.
 *
 * Errors: every status of attn_fwd_splitkv except ATTN_ERR_WORKSPACE, plus
 * ATTN_ERR_SCRATCH when attn_splitkv_workspace_bytes(B, H, Nq, Nk, D, num_splits)
 * exceeds ATTN_NOALLOC_SCRATCH_BYTES (nothing is launched); ATTN_ERR_HIP if the
 * scratch address cannot be obtained.  Nothing in the scratch must start at zero
 * (every partial result is written before it is read).  All calls on one device
 * share its scratch: calls that may overlap on that device (different streams,
 * or other threads) race and must be ordered by the caller.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int Nq, int Nk, int D, float scale, int causal,
                             const int32_t* kv_lens, int num_splits, void* stream);

/* attn_strerror -- a static, NUL-terminated description of a status code. */
const char* attn_strerror(int status);

/* attn_abi_version -- version of this ABI (incremented on incompatible change). */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_89_ATTN_H */
