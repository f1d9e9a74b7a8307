// Tile schedules shared by the kernels: which key (or query) tiles a
// workgroup visits under dense, causal and block-sparse masks.
//
// Block-sparse attention skips every zero block of the mask entirely, so its
// IO and run time shrink with the number of nonzero blocks (block-sparse
// FlashAttention, abstract of "FlashAttention: Fast and Memory-Efficient
// Exact Attention with IO-Awareness").
#pragma once

#include "fa_device.h"

namespace fa {

// Compacts, in ascending order, the indices idx in [lo, hi) whose mask byte
// mask[base + idx * stride] is nonzero into list[0 .. count).  All NT
// threads of the workgroup must call it; it returns the count to every
// thread.  `wcount` is NW ints of LDS scratch.
template <int NT>
__device__ __forceinline__ int compact_mask_run(const uint8_t* mask, size_t base, size_t stride,
                                                int lo, int hi, int* list, int* wcount) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  int cnt = 0;
  __syncthreads();  // earlier readers of list / wcount are done
  for (int b0 = lo; b0 < hi; b0 += NT) {
    const int idx = b0 + tid;
    const bool f = idx < hi && mask[base + (size_t)idx * stride] != 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(f);
    const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    (void)lane;
    if ((tid & 63) == 0) wcount[w] = __popcll(bal);
    __syncthreads();
    int off = cnt;
    for (int u = 0; u < w; ++u) off += wcount[u];
    if (f) list[off + pos] = idx;
    for (int u = 0; u < NW; ++u) cnt += wcount[u];
    __syncthreads();
  }
  return cnt;
}

}  // namespace fa
