// Work assignment of the decode kernels, computed on the device from the
// actual context lengths by every workgroup (the merge kernel reads the run
// length back from the workspace header).
//
// Partitions are the split granularity; one wave streams a run of `span`
// consecutive partitions of one (sequence, kv head) and merges it online
// (the running-max rescaling is itself an exact log-sum-exp merge), so one
// record covers a run.  span is the smallest whole number of partitions
// that leaves at most `target_waves` (run, kv head) items over the batch:
//   items(span) = sum_b ceil(n_b / span) * kv_heads <= target_waves,
//   n_b = ceil(L_b / P);
// items(s) does not grow with s, so it is found by bisection.  Long
// sequences therefore get long runs, and a batch of short or mixed lengths
// keeps span 1.  When batch * kv_heads alone reaches the target, span is 1
// (the library then normally picks one partition per sequence instead).
//
// Items are (run, head group) pairs over the real runs only, numbered
// sequence by sequence: sequence b owns runs [R_b, R_b + runs_b), R_b the
// prefix sum of runs over the sequences before it, and head groups are
// fastest.  Workgroup i takes item i; consecutive workgroups are dealt
// round-robin to the eight XCDs.  (Measured on MI355X: as fast as numbering
// by run index first on uniform lengths and 3 % faster on mixed lengths;
// dealing each XCD a contiguous share of the items was 6-19 % slower.)
// There are at most target_waves / wpg items of wpg-head workgroups when
// batch * kv_heads is below the target; the host launches that many
// workgroups and those left without an item exit.
#pragma once

#include "pa_internal.h"

namespace pa {

struct RunSlot {
  int span;   // partitions per run
  int b;      // sequence, or -1: no item for this workgroup
  int ridx;   // run index within the sequence
  int grp;    // head group (kv heads grp*wpg .. grp*wpg+wpg-1)
};

__device__ inline int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return __builtin_amdgcn_readfirstlane(x);
}

// Item of this workgroup.  Must be called by all 64 lanes of each wave; the
// result is wave-uniform.  In direct mode (one partition covers every
// context) the runs are the sequences themselves, empty or invalid ones
// included: the kernel writes their rows.
__device__ inline RunSlot locate_run(const DecodeParams& p, int groups) {
  RunSlot r{1, -1, 0, (int)(blockIdx.x % groups)};
  const int item = blockIdx.x / groups;      // run number, head groups fastest
  if (p.direct) {
    if (item < p.batch) r.b = item;
    return r;
  }
  const int lane = threadIdx.x & 63;
  const int P = p.partition_size;
  const int max_part = (p.max_context_len + P - 1) / P;
  auto parts = [&](int b) {                  // partitions of sequence b (0 if invalid)
    if (b >= p.batch) return 0;
    const int L = p.context_lens[b] - p.token_offset;
    return (L > 0 && L <= p.max_context_len) ? (L + P - 1) / P : 0;
  };
  const int n0 = parts(lane);                // batches of up to 64 need one load
  auto parts_of = [&](int b0) { return b0 == 0 ? n0 : parts(b0 + lane); };
  // span: the smallest run length (in partitions) that leaves at most
  // target_waves (run, kv head) items; items(s) does not grow with s, and at
  // s = max_part every sequence is one run (batch * kv_heads < target).
  auto items = [&](int s) {
    long long runs = 0;
    for (int b0 = 0; b0 < p.batch; b0 += 64) runs += wave_sum((parts_of(b0) + s - 1) / s);
    return runs * p.kv_heads;
  };
  int span = 1;
  if ((long long)p.batch * p.kv_heads < p.target_waves && items(1) > p.target_waves) {
    int lo = 1, hi = max_part;               // items(lo) > target >= items(hi)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (items(mid) <= p.target_waves) hi = mid; else lo = mid;
    }
    span = hi;
  }
  r.span = span = __builtin_amdgcn_readfirstlane(span);
  auto runs_of = [&](int b0) { return (parts_of(b0) + span - 1) / span; };

  // the sequence whose runs hold `item`: prefix sum of runs over the lanes
  int base = 0;                              // runs of the sequences before chunk b0
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int runs = runs_of(b0);
    int incl = runs;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const int chunk = __builtin_amdgcn_readlane(incl, 63);
    if (item < base + chunk) {
      // lanes whose runs all lie before the item form a prefix; the next
      // lane owns it
      const int k = (int)__builtin_popcountll(__ballot(base + incl <= item));
      r.b = b0 + k;
      r.ridx = item - base - (__builtin_amdgcn_readlane(incl, k) -
                              __builtin_amdgcn_readlane(runs, k));
      return r;
    }
    base += chunk;
  }
  return r;                                  // past the last run: b = -1
}

}  // namespace pa
