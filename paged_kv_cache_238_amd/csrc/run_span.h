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
// and items map to (partition, sequence) directly, without reading lengths
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
  int len;    // context_lens[b] - token_offset when the search read it, else -1
};

// Cross-lane steps on the VALU (DPP and gfx950's permlane swaps) rather
// than LDS lane shuffles: the run search is on every workgroup's start-up
// path, where each shuffle's LDS round trip would add to the latency.
__device__ inline int dpp(int x, int ctrl) {
  switch (ctrl) {   // the control must be a constant
    case 0xB1: return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true);    // quad lanes ^1
    case 0x4E: return __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true);    // quad lanes ^2
    case 0x124: return __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, true);  // row rotate 4
    case 0x128: return __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, true);  // row rotate 8
    case 0x111: return __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row shift 1
    case 0x112: return __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row shift 2
    case 0x114: return __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row shift 4
    default: return __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);     // row shift 8
  }
}

// Sum over the wave, wave-uniform result.
__device__ inline int wave_sum(int x) {
  x += dpp(x, 0xB1);
  x += dpp(x, 0x4E);                         // every lane: its quad's sum
  x += dpp(x, 0x124);
  x += dpp(x, 0x128);                        // its row of 16
  const auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  x = (int)(a[0] + a[1]);                    // rows 0+1, 2+3
  const auto c = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return __builtin_amdgcn_readfirstlane((int)(c[0] + c[1]));
}

// Inclusive prefix sum over the lanes (lane i: x_0 + ... + x_i).
__device__ inline int wave_scan(int x) {
  x += dpp(x, 0x111);
  x += dpp(x, 0x112);
  x += dpp(x, 0x114);
  x += dpp(x, 0x118);                        // within each row of 16
  // last lane of row 0 (2) into row 1 (3), then of row 1 into rows 2 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
  return x;
}

// Item of this workgroup.  Must be called by all 64 lanes of each wave; the
// result is wave-uniform.  In direct mode (one partition covers every
// context) the runs are the sequences themselves, empty or invalid ones
// included: the kernel writes their rows.
__device__ inline RunSlot locate_run(const DecodeParams& p, int groups) {
  RunSlot r{1, -1, 0, (int)(blockIdx.x % groups), -1};
  const int item = blockIdx.x / groups;      // run number, head groups fastest
  if (p.direct) {
    if (item < p.batch) r.b = item;
    return r;
  }
  if ((long long)p.batch * p.kv_heads >= p.target_waves) {
    // Pairs alone fill the GPU: one partition per run, numbered partition
    // index first (the host launches n_part * batch items); a workgroup
    // whose sequence has no such partition finds an empty run and exits.
    // No lengths are scanned, so the prologue does not grow with the batch.
    r.ridx = item / p.batch;
    r.b = item % p.batch;
    return r;
  }
  const int lane = threadIdx.x & 63;
  const int P = p.partition_size;
  const int max_part = (p.max_context_len + P - 1) / P;
  auto length = [&](int b) { return b < p.batch ? p.context_lens[b] - p.token_offset : 0; };
  auto parts_in = [&](int L) {               // partitions of a length (0 if invalid)
    return (L > 0 && L <= p.max_context_len) ? (L + P - 1) / P : 0;
  };
  const int len0 = length(lane);             // batches of up to 64 need one load
  const int n0 = parts_in(len0);
  auto parts_of = [&](int b0) { return b0 == 0 ? n0 : parts_in(length(b0 + lane)); };
  // span: the smallest run length (in partitions) that leaves at most
  // target_waves (run, kv head) items; items(s) does not grow with s, and at
  // s = max_part every sequence is one run (batch * kv_heads < target).
  auto items = [&](int s) {
    long long runs = 0;
    for (int b0 = 0; b0 < p.batch; b0 += 64) runs += wave_sum((parts_of(b0) + s - 1) / s);
    return runs * p.kv_heads;
  };
  int span = 1;
  if (items(1) > p.target_waves) {
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
    const int incl = wave_scan(runs);
    const int chunk = __builtin_amdgcn_readlane(incl, 63);
    if (item < base + chunk) {
      // lanes whose runs all lie before the item form a prefix; the next
      // lane owns it
      const int k = (int)__builtin_popcountll(__ballot(base + incl <= item));
      r.b = b0 + k;
      // the owner's length, already loaded: the kernel need not read it again
      r.len = __builtin_amdgcn_readlane(b0 == 0 ? len0 : length(b0 + lane), k);
      r.ridx = item - base - (__builtin_amdgcn_readlane(incl, k) -
                              __builtin_amdgcn_readlane(runs, k));
      return r;
    }
    base += chunk;
  }
  return r;                                  // past the last run: b = -1
}

}  // namespace pa
