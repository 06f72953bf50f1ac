// mfma_schedule.hpp -- instruction order of a run of MFMAs fed from LDS, for the four-wave
// kernels (attn_fwd_bf16_4w.hip, attn_fwd_fp8.hip).
#pragma once

namespace attn89 {

// Issue order of NM MFMAs with R fragment reads each: the reads of the first PF MFMAs
// first, then the reads of one more MFMA after every MFMA, so each fragment is requested
// PF MFMAs before it is used; NVM global requests (the next tile's DMA) go between the
// MFMAs, as evenly as they fit.  Left to itself the compiler issues each read just
// before its MFMA and the requests in one burst (a request the memory pipeline cannot
// take yet stalls the wave, which costs least while MFMAs are queued).  Call it right
// after the code that issues the MFMAs, in the same basic block.
template <int NM, int R, int NVM, int PF>
__device__ __forceinline__ void schedule_mfma_run() {
  constexpr int kPf = NM < PF ? NM : PF;
  constexpr int ITER = NM - kPf;
  constexpr int VMI = ITER > 0 ? (NVM + ITER - 1) / ITER : 0;
  __builtin_amdgcn_sched_group_barrier(0x100, R * kPf, 0);       // LDS reads
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);           // the reads of a later one
    if (VMI > 0 && i * VMI < NVM)
      __builtin_amdgcn_sched_group_barrier(0x020, VMI, 0);       // global requests
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kPf, 0);
}

}  // namespace attn89
