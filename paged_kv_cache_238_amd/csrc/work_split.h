// Work assignment of the decode kernels, computed on the device from the
// actual context lengths by every workgroup (the merge kernel reads the
// record counts back from the workspace header).
//
// Three modes, in the order the library picks them:
//
// * Direct (one partition covers every context): workgroup item = sequence;
//   the wave streams the whole context and writes the output row itself.
//
// * Partition items (batch * kv_heads alone reaches the wave target): item =
//   (partition, sequence), partition first; the host launches n_part * batch
//   items and those past a sequence's end exit.  No lengths are scanned, so
//   the start-up does not grow with the batch.  Record r of a row covers
//   partition r (header[0] = 1).
//
// * Balanced chunks (otherwise).  The blocks of all sequences are laid end
//   to end, sequence by sequence: sequence b owns flattened blocks
//   [F_b, F_b + nb_b), nb_b = ceil(L_b / 16) (0 for an empty or invalid
//   length), F_b the prefix sum.  That line of T blocks is cut into chunks
//   of C blocks,
//     C = max(P / 16, ceil(T / K)),   K = target_waves / kv_heads,
//   so there are at most K chunks and every wave (one per chunk and kv head)
//   streams the same number of blocks, C, give or take the last chunk.  A
//   chunk that crosses sequence boundaries is streamed as consecutive
//   segments, one record each; the running-max rescaling makes each record
//   an exact log-sum-exp merge of its blocks.  Record r of sequence b comes
//   from chunk floor(F_b / C) + r, so b has
//     n_b = floor((F_b + nb_b - 1) / C) - floor(F_b / C) + 1 <= ceil(nb_b / C) + 1
//   records (at most n_part + 1, since C >= P / 16); the wave that streams
//   b's first block stores n_b in header[kCountsAt + b] (header[0] = 0).
//   With runs cut at sequence starts instead, a mixed-length batch left its
//   waves between a fraction of a run and a whole run long, and the kernel
//   lasted as long as the whole ones.
//
// Items are (chunk, head group) with head groups fastest; consecutive
// workgroups are dealt round-robin to the eight XCDs.  The host launches
// K * groups workgroups (fewer when the partitions bound the chunks) and
// those without a chunk exit.
#pragma once

#include "pa_internal.h"

namespace pa {

struct Segment {
  int b;      // sequence, or -1: no item for this workgroup
  int len;    // seq_len(p, b) when already read, else -1
  int j0;     // first block of the segment within the sequence's table row
  int nblk;   // blocks of the segment (the kernel clamps by the length)
  int rec;    // record index within the (sequence, head) row
  int grp;    // head group (kv heads grp*wpg .. grp*wpg+wpg-1)
  // Balanced chunks only (end < 0 otherwise):
  int F;      // flattened index of sequence b's first block
  int nb;     // blocks of sequence b
  int end;    // flattened end of the chunk (exclusive)
  int C;      // chunk length in blocks
  int lane_len;   // per lane, not uniform: the length of sequence `lane`
                  // (balanced chunks over batches of up to 64 sequences)
};

// Cross-lane steps on the VALU (DPP and gfx950's permlane swaps) rather
// than LDS lane shuffles: the search is on every workgroup's start-up path,
// where each shuffle's LDS round trip would add to the latency.
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

// Blocks of a sequence of length L (0 when empty or outside the contract,
// so such a sequence owns no chunk and the merge writes its row).
__device__ inline int blocks_of(const DecodeParams& p, int L) {
  return (L > 0 && L <= p.max_context_len) ? (L + kBlockTokens - 1) / kBlockTokens : 0;
}

// First segment of workgroup `wg` of the launch's partition work.  Must be
// called by all 64 lanes of each wave; the result is wave-uniform.
__device__ inline Segment locate_work(const DecodeParams& p, int groups, int wg) {
  Segment s{-1, -1, 0, 0, 0, wg % groups, 0, 0, -1, 0, 0};
  const int item = wg / groups;              // head groups fastest
  const int P = p.partition_size;
  if (p.direct) {                            // empty or invalid sequences included
    if (item < p.batch) {
      s.b = item;
      s.nblk = p.max_blocks;
    }
    return s;
  }
  if ((long long)p.batch * p.kv_heads >= p.target_waves) {
    s.rec = item / p.batch;                  // partition
    s.b = item % p.batch;
    s.j0 = s.rec * (P / kBlockTokens);
    s.nblk = P / kBlockTokens;
    return s;
  }
  const int lane = threadIdx.x & 63;
  auto length = [&](int b) { return b < p.batch ? seq_len(p, b) : 0; };
  const int len0 = length(lane);             // batches of up to 64 need one load
  const int nb0 = blocks_of(p, len0);
  auto nb_of = [&](int b0) { return b0 == 0 ? nb0 : blocks_of(p, length(b0 + lane)); };
  int T = 0;
  for (int b0 = 0; b0 < p.batch; b0 += 64) T += wave_sum(nb_of(b0));
  const int K = max(1, p.target_waves / p.kv_heads);
  const int C = max(P / kBlockTokens, (T + K - 1) / K);
  const int start = item * C;
  if (T == 0 || item >= (T + C - 1) / C) return s;
  s.C = C;
  s.end = min(start + C, T);
  s.lane_len = len0;
  // the sequence holding flattened block `start`: prefix sum over the lanes
  int base = 0;                              // blocks of the sequences before chunk b0
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int nb = nb_of(b0);
    const int incl = wave_scan(nb);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (start < base + total) {
      // lanes whose blocks all lie before `start` form a prefix; the next
      // lane (a sequence with blocks) owns it
      const int k = (int)__builtin_popcountll(__ballot(base + incl <= start));
      s.b = b0 + k;
      s.nb = __builtin_amdgcn_readlane(nb, k);
      s.F = base + __builtin_amdgcn_readlane(incl, k) - s.nb;
      s.len = __builtin_amdgcn_readlane(b0 == 0 ? len0 : length(b0 + lane), k);
      s.j0 = start - s.F;
      s.nblk = min(s.F + s.nb, s.end) - start;
      s.rec = item - s.F / C;
      return s;
    }
    base += total;
  }
  return s;                                  // not reached: start < T
}

// Next segment of a balanced chunk: the following sequence with blocks, if
// the chunk reaches it.  Wave-uniform.  Batches of up to 64 take the length
// from the lanes that locate_work loaded, so the switch waits on no memory
// read before the table ids.
__device__ inline bool next_segment(const DecodeParams& p, Segment& s) {
  if (s.end < 0) return false;
  const int F = s.F + s.nb;
  if (F >= s.end) return false;
  int b = s.b, L = 0, nb = 0;
  while (nb == 0 && b + 1 < p.batch) {
    ++b;
    L = p.batch <= 64 ? __builtin_amdgcn_readlane(s.lane_len, b) : seq_len(p, b);
    nb = blocks_of(p, L);
  }
  if (nb == 0) return false;                 // not reached: F < end <= T
  s.b = b;
  s.len = L;
  s.F = F;
  s.nb = nb;
  s.j0 = 0;
  s.nblk = min(nb, s.end - F);
  s.rec = 0;                                 // the chunk holds b's first block
  return true;
}

// Balanced chunks: the segment holding a sequence's first block stores the
// sequence's record count for the merge (one lane of the workgroup's first
// head group).
__device__ inline void note_record_count(const DecodeParams& p, const Segment& s, bool writer) {
  if (s.end >= 0 && s.j0 == 0 && s.grp == 0 && writer)
    p.header[kCountsAt + s.b] = (s.F + s.nb - 1) / s.C - s.F / s.C + 1;
}

}  // namespace pa
