// attn_api.hip -- the C ABI of include/attn.h: argument checks, then dispatch.
//
// Every check runs before anything is launched, so an error status means no
// kernel ran and no output was written.  kv_lens is device memory and is not read
// here (that would need a synchronisation); the kernels clamp its entries.

#include <math.h>

#include <mutex>

#include "../../include/attn.h"
#include "common.hpp"
#include "launch.hpp"

namespace {

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

int check_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 int B, int H, int Nq, int Nk, int D, float scale, const int32_t* kv_lens,
                 size_t elem_bytes) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  size_t bh = 0, nq = 0, nk = 0, bytes = 0;
  if (__builtin_mul_overflow((size_t)B, (size_t)H, &bh)) return ATTN_ERR_SHAPE;
  if (__builtin_mul_overflow(bh, (size_t)Nq, &nq)) return ATTN_ERR_SHAPE;
  if (__builtin_mul_overflow(bh, (size_t)Nk, &nk)) return ATTN_ERR_SHAPE;
  if (__builtin_mul_overflow(nq > nk ? nq : nk, (size_t)D * elem_bytes, &bytes))
    return ATTN_ERR_SHAPE;
  if (bh > 0x7fffffffULL) return ATTN_ERR_TOO_LARGE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return ATTN_ERR_ALIGN;
  if (!aligned(lse, 4) || (kv_lens && !aligned(kv_lens, 4))) return ATTN_ERR_ALIGN;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  return ATTN_OK;
}

attn89::FwdArgs make_args(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int Nq, int Nk, float scale, int causal,
                          const int32_t* kv_lens) {
  attn89::FwdArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.kv_lens = kv_lens;
  a.B = B;
  a.H = H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.causal = causal ? 1 : 0;
  const float c = scale * attn89::kLog2e;
  if (scale > 0.f) {
    a.c_exp = c;
    a.c_pre = 1.f;
    a.pre_scale = 0;
  } else {
    a.c_exp = 1.f;
    a.c_pre = c;
    a.pre_scale = 1;
  }
  return a;
}

// Which bf16 forward kernel attn_fwd launches (attn_fwd_select_kernel).
int g_bf16_kernel = ATTN_KERNEL_AUTO;

// Compute units of the current device, cached per device.
int num_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;
  if (dev < 64) cache[dev] = n;
  return n;
}

// The 8-wave ping-pong kernel (one 256-row workgroup per CU) is the faster one once
// its blocks are full (Nq >= 256) and its grid covers every CU; below that, and for
// D = 64 (where the softmax, not the matrix work, bounds a tile), the 4-wave kernel
// with smaller blocks and twice as many workgroups wins.  When even its grid gives
// no CU a second workgroup, the time is the longest block's key loop, and the key
// groups variant halves that loop.
int pick_bf16_kernel(int B, int H, int Nq, int D) {
  if (g_bf16_kernel != ATTN_KERNEL_AUTO) return g_bf16_kernel;
  const long long pp_grid = (long long)((Nq + 255) / 256) * B * H;
  if (D == 128 && Nq >= 256 && pp_grid >= num_cus()) return ATTN_KERNEL_PINGPONG;
  const long long grid4 = (long long)((Nq + 127) / 128) * B * H;
  return grid4 <= num_cus() ? ATTN_KERNEL_KEYGROUPS : ATTN_KERNEL_FOURWAVE;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int Nq, int Nk, int D, float scale, int causal, const int32_t* kv_lens,
             void* stream) {
  int st = check_common(q, k, v, o, lse, B, H, Nq, Nk, D, scale, kv_lens, 2);
  if (st != ATTN_OK) return st;
  // one head of q or k/v (plus a tile of slack) must be addressable with 32-bit
  // byte offsets by the kernel's buffer loads
  if (((size_t)Nq + 256) * D * 2 >= ((size_t)1 << 31) ||
      ((size_t)Nk + 256) * D * 2 >= ((size_t)1 << 31))
    return ATTN_ERR_TOO_LARGE;
  attn89::FwdArgs a = make_args(q, k, v, o, lse, B, H, Nq, Nk, scale, causal, kv_lens);
  const int which = pick_bf16_kernel(B, H, Nq, D);
  if (which == ATTN_KERNEL_PINGPONG)
    return attn89::launch_attn_fwd_bf16_pp(a, D, (hipStream_t)stream);
  return attn89::launch_attn_fwd_bf16_4w(a, D, (hipStream_t)stream,
                                         which == ATTN_KERNEL_KEYGROUPS ? 2 : 1);
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                 int H, int Nq, int Nk, int D, float scale, float q_descale, float k_descale,
                 float v_descale, int causal, const int32_t* kv_lens, void* stream) {
  int st = check_common(q, k, v, o, lse, B, H, Nq, Nk, D, scale, kv_lens, 1);
  if (st != ATTN_OK) return st;
  for (float d : {q_descale, k_descale, v_descale})
    if (!(isfinite(d) && d > 0.f)) return ATTN_ERR_SCALE;
  const float s_eff = scale * q_descale * k_descale;   // the score scale, in fp32
  if (!isfinite(s_eff)) return ATTN_ERR_SCALE;
  if (((size_t)Nq + 256) * D >= ((size_t)1 << 31) || ((size_t)Nk + 256) * D >= ((size_t)1 << 31))
    return ATTN_ERR_TOO_LARGE;
  attn89::FwdArgs a = make_args(q, k, v, o, lse, B, H, Nq, Nk, s_eff, causal, kv_lens);
  // FP8: the 4-wave kernel unless the ping-pong kernel is requested explicitly.  The
  // FP8 softmax outlasts the FP8 matrix phase, and the ping-pong lock-step then leaves
  // the matrix cores idle (B=1 H=32 N=8192 causal: 0.402 ms against 0.360 ms).
  if (g_bf16_kernel == ATTN_KERNEL_PINGPONG)
    return attn89::launch_attn_fwd_fp8_pp(a, D, v_descale, (hipStream_t)stream);
  return attn89::launch_attn_fwd_fp8(a, D, v_descale, (hipStream_t)stream);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int H,
                    int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int D,
                    float scale, int causal, void* stream) {
  if (!cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_NULL;
  if (!aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4)) return ATTN_ERR_ALIGN;
  if (max_seqlen_q < 1 || max_seqlen_k < 1) return ATTN_ERR_SHAPE;
  // the common checks on the packed tensors: one "batch" of total_q / total_k rows of H*D
  int st = check_common(q, k, v, o, lse, 1, H, total_q, total_k, D, scale, nullptr, 2);
  if (st != ATTN_OK) return st;
  if (B < 1) return ATTN_ERR_SHAPE;
  // per-sequence byte offsets (rows H*D apart, plus a tile of slack) stay below 2^31
  const size_t row_bytes = (size_t)H * D * 2;
  if (((size_t)max_seqlen_q + 256) * row_bytes >= ((size_t)1 << 31) ||
      ((size_t)max_seqlen_k + 256) * row_bytes >= ((size_t)1 << 31))
    return ATTN_ERR_TOO_LARGE;
  if ((long long)((max_seqlen_q + 127) / 128) * B * H > 0x7fffffffLL) return ATTN_ERR_TOO_LARGE;
  attn89::FwdArgs a = make_args(q, k, v, o, lse, B, H, max_seqlen_q, max_seqlen_k, scale,
                                causal, nullptr);
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  return attn89::launch_attn_fwd_bf16_4w_varlen(a, D, (hipStream_t)stream);
}

int attn_fwd_select_kernel(int which) {
  if (which != ATTN_KERNEL_AUTO && which != ATTN_KERNEL_PINGPONG &&
      which != ATTN_KERNEL_FOURWAVE && which != ATTN_KERNEL_KEYGROUPS)
    return ATTN_ERR_UNSUPPORTED;
  const int prev = g_bf16_kernel;
  g_bf16_kernel = which;
  return prev;
}

int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                 int H, int Nq, int Nk, int D, float scale, int causal, const int32_t* kv_lens,
                 void* stream) {
  int st = check_common(q, k, v, o, lse, B, H, Nq, Nk, D, scale, kv_lens, 4);
  if (st != ATTN_OK) return st;
  attn89::FwdArgs a = make_args(q, k, v, o, lse, B, H, Nq, Nk, scale, causal, kv_lens);
  return attn89::launch_attn_fwd_f32(a, D, (hipStream_t)stream);
}

size_t attn_materialized_workspace_bytes(int B, int H, int Nq, int Nk) {
  attn89::MatLayout lay;
  if (!attn89::materialized_layout(B, H, Nq, Nk, &lay)) return 0;
  return lay.total;
}

int attn_materialized(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int Nq, int Nk, int D, float scale, int causal,
                      const int32_t* kv_lens, void* workspace, size_t workspace_bytes,
                      void* stream) {
  int st = check_common(q, k, v, o, lse, B, H, Nq, Nk, D, scale, kv_lens, 2);
  if (st != ATTN_OK) return st;
  attn89::MatLayout lay;
  if (!attn89::materialized_layout(B, H, Nq, Nk, &lay)) return ATTN_ERR_SHAPE;
  if (!workspace || workspace_bytes < lay.total || !aligned(workspace, 256))
    return ATTN_ERR_WORKSPACE;
  attn89::FwdArgs a = make_args(q, k, v, o, lse, B, H, Nq, Nk, scale, causal, kv_lens);
  return attn89::launch_attn_materialized(a, D, scale, workspace, lay, (hipStream_t)stream);
}

// workspace of attn_fwd_splitkv: o_part (fp32) then lse_part, each 256-aligned
static bool splitkv_layout(int B, int H, int Nq, int Nk, int D, int num_splits, int* splits,
                           int* chunk, size_t* lse_off, size_t* total) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (D != 64 && D != 128)) return false;
  *splits = attn89::splitkv_plan(B, H, Nq, Nk, num_splits, num_cus(), chunk);
  size_t rows = 0, o_elems = 0;
  if (__builtin_mul_overflow((size_t)B * (size_t)H, (size_t)Nq, &rows)) return false;
  if (__builtin_mul_overflow(rows * (size_t)*splits, (size_t)D, &o_elems)) return false;
  if (o_elems > ((size_t)1 << 56)) return false;
  *lse_off = (o_elems * 4 + 255) / 256 * 256;
  *total = *lse_off + (rows * (size_t)*splits * 4 + 255) / 256 * 256;
  return true;
}

int attn_splitkv_num_splits(int B, int H, int Nq, int Nk, int num_splits) {
  int chunk = 0;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return ATTN_ERR_SHAPE;
  return attn89::splitkv_plan(B, H, Nq, Nk, num_splits, num_cus(), &chunk);
}

size_t attn_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int D, int num_splits) {
  int splits = 0, chunk = 0;
  size_t lse_off = 0, total = 0;
  if (!splitkv_layout(B, H, Nq, Nk, D, num_splits, &splits, &chunk, &lse_off, &total)) return 0;
  return total;
}

}  // extern "C"

namespace {

// The checks and the launch of attn_fwd_splitkv and attn_fwd_splitkv_noalloc.  When
// `need` is not null the workspace is not checked: the caller learns the bytes the
// problem needs through it and passes its own buffer afterwards.
int splitkv_checked(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int Nq, int Nk, int D, float scale, int causal,
                    const int32_t* kv_lens, int num_splits, void* workspace,
                    size_t workspace_bytes, void* stream, size_t* need) {
  int st = check_common(q, k, v, o, lse, B, H, Nq, Nk, D, scale, kv_lens, 2);
  if (st != ATTN_OK) return st;
  if (((size_t)Nq + 256) * D * 2 >= ((size_t)1 << 31) ||
      ((size_t)Nk + 256) * D * 2 >= ((size_t)1 << 31))
    return ATTN_ERR_TOO_LARGE;
  int splits = 0, chunk = 0;
  size_t lse_off = 0, total = 0;
  if (!splitkv_layout(B, H, Nq, Nk, D, num_splits, &splits, &chunk, &lse_off, &total))
    return ATTN_ERR_SHAPE;
  if ((long long)((Nq + 127) / 128) * B * H * splits > 0x7fffffffLL) return ATTN_ERR_TOO_LARGE;
  if (need) {
    *need = total;
    return ATTN_OK;
  }
  if (!workspace || workspace_bytes < total || !aligned(workspace, 256))
    return ATTN_ERR_WORKSPACE;
  attn89::FwdArgs a = make_args(q, k, v, o, lse, B, H, Nq, Nk, scale, causal, kv_lens);
  a.n_splits = splits;
  a.kv_chunk = chunk;
  a.o_part = (float*)workspace;
  a.lse_part = (float*)((char*)workspace + lse_off);
  return attn89::launch_attn_splitkv(a, D, (hipStream_t)stream);
}

// The fixed scratch of attn_fwd_splitkv_noalloc: one copy per device, held from the
// library's load until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress, looked up once per device (with that device current) and kept.
constexpr size_t kScratchBytes = (size_t)ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, or null (status in *st).
void* scratch_address(int* st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *st = ATTN_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      *st = ATTN_ERR_HIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *st = ATTN_OK;
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int Nq, int Nk, int D, float scale, int causal,
                     const int32_t* kv_lens, int num_splits, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return splitkv_checked(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, kv_lens, num_splits,
                         workspace, workspace_bytes, stream, nullptr);
}

int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int Nq, int Nk, int D, float scale, int causal,
                             const int32_t* kv_lens, int num_splits, void* stream) {
  size_t need = 0;
  int st = splitkv_checked(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, kv_lens,
                           num_splits, nullptr, 0, stream, &need);
  if (st != ATTN_OK) return st;
  if (need > kScratchBytes) return ATTN_ERR_SCRATCH;
  void* ws = scratch_address(&st);
  if (!ws) return st;
  return splitkv_checked(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, kv_lens, num_splits,
                         ws, kScratchBytes, stream, nullptr);
}

size_t attn_partial_workspace_bytes(int B, int H, int Nq, int Nk) {
  attn89::MatLayout lay;
  if (!attn89::materialized_layout(B, H, Nq, Nk, &lay)) return 0;
  const size_t p_bytes = lay.total - lay.p_offset;   // P alone: B*H*Nq*ld*2
  return (p_bytes + 255) / 256 * 256;
}

int attn_partial(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                 int H, int Nq, int Nk, int D, float scale, int causal,
                 const int32_t* kv_lens, void* workspace, size_t workspace_bytes,
                 void* stream) {
  int st = check_common(q, k, v, o, lse, B, H, Nq, Nk, D, scale, kv_lens, 2);
  if (st != ATTN_OK) return st;
  if (((size_t)Nq + 256) * D * 2 >= ((size_t)1 << 31) ||
      ((size_t)Nk + 256) * D * 2 >= ((size_t)1 << 31))
    return ATTN_ERR_TOO_LARGE;
  if ((long long)B * H > 65535) return ATTN_ERR_TOO_LARGE;   // grid of the P V launch
  attn89::MatLayout lay;
  if (!attn89::materialized_layout(B, H, Nq, Nk, &lay)) return ATTN_ERR_SHAPE;
  if (!workspace || workspace_bytes < attn_partial_workspace_bytes(B, H, Nq, Nk) ||
      !aligned(workspace, 256))
    return ATTN_ERR_WORKSPACE;
  attn89::FwdArgs a = make_args(q, k, v, o, lse, B, H, Nq, Nk, scale, causal, kv_lens);
  return attn89::launch_attn_partial(a, D, lay.ld, (unsigned short*)workspace,
                                     (hipStream_t)stream);
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, H, Nq and Nk must be >= 1 and the sizes must fit 64 bits";
    case ATTN_ERR_UNSUPPORTED: return "head dimension must be 64 or 128";
    case ATTN_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned; lse, kv_lens 4-byte";
    case ATTN_ERR_SCALE: return "scale must be finite";
    case ATTN_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case ATTN_ERR_HIP: return "the HIP runtime reported a launch error";
    case ATTN_ERR_TOO_LARGE: return "problem exceeds the kernel launch limits";
    case ATTN_ERR_SCRATCH:
      return "problem needs more than the fixed scratch of attn_fwd_splitkv_noalloc";
    default: return "unknown status";
  }
}

int attn_abi_version(void) { return 2; }

}  // extern "C"
