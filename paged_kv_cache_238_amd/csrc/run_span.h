// Run length of the decode kernels, computed on the device from
// the actual context lengths, identically by the partition kernel and the
// merge kernel.
//
// Partitions are the split granularity; one wave streams a run of `span`
// consecutive partitions of one (sequence, kv head) and merges them online
// (the running-max rescaling is itself an exact log-sum-exp merge), so one
// record covers a run.  span is the largest power of two that still leaves
// at least `target_waves` runs over the whole batch:
//   sum_b ceil(n_b / span) * kv_heads >= target_waves,  n_b = ceil(L_b / P).
// Long sequences therefore get long runs, and a batch of short or mixed
// lengths keeps span 1.  When batch * kv_heads alone reaches the target no
// length is read and span is 1.
#pragma once

#include "pa_internal.h"

namespace pa {

// Must be called by all 64 lanes of a wave; the result is wave-uniform.
__device__ inline int run_span(const int32_t* context_lens, int batch, int kv_heads,
                               int max_context_len, int partition_size, int target_waves) {
  if ((long long)batch * kv_heads >= target_waves) return 1;
  const int lane = threadIdx.x & 63;
  const int max_part = (max_context_len + partition_size - 1) / partition_size;
  auto parts = [&](int b) {                  // partitions of sequence b (0 if invalid)
    if (b >= batch) return 0;
    const int L = context_lens[b];
    return (L > 0 && L <= max_context_len) ? (L + partition_size - 1) / partition_size : 0;
  };
  const int n0 = parts(lane);                // batches of up to 64 need one load
  int span = 1;
  for (int s = 2; s <= max_part; s *= 2) {
    long long runs = 0;
    for (int b0 = 0; b0 < batch; b0 += 64) {
      const int n = b0 == 0 ? n0 : parts(b0 + lane);
      int r = (n + s - 1) / s;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) r += __shfl_xor(r, off);
      runs += r;
    }
    if (runs * kv_heads < target_waves) break;
    span = s;
  }
  return __builtin_amdgcn_readfirstlane(span);
}

}  // namespace pa
