// Paged-attention decode, split-K partition kernel (VALU form) for gfx950,
// used for query-head groups of 1 or 2 (larger groups use the matrix-core
// kernel in decode_mfma.hip).
//
// Work split (as in the matrix-core kernel): a workgroup holds up to four
// waves for consecutive kv heads of one work item - a balanced chunk of
// blocks sized on the device from the actual context lengths
// (work_split.h), a partition, or a whole sequence; each wave streams its
// head's blocks of the item, merges them online and writes one record (max
// reference, sum, unnormalised output) per sequence the item reaches, for
// the log-sum-exp merge kernel, or the final fp16 row when one partition
// covers the context.
//
// Method: the zskr.cn article on ATB's PagedAttention, section
// "PagedAttention 的 Attention 计算修改" - per-page gather through the page
// table, dot of Q with each K row, running max with rescaling of the
// accumulator, V accumulation, final normalisation.  Differences from that
// listing: the running max is updated before the new term's exponent is
// taken, the max starts at -inf, a softmax scale is applied, accumulation is
// fp32, the output is indexed by head, and tail slots are masked.  The page
// table slice is read once per wave and held one id per lane (section
// "踩坑一").  Query heads h = g*G .. g*G+G-1 share kv head g (discosf.com
// article "KV Cache 优化与显存管理", section "二、优化方向").
//
// Lane layout: a K/V row (one token, one kv head) of D elements is split
// over D/8 lanes holding 8 consecutive elements each (16 B for fp16, 8 B for
// int8), so one wave-wide load covers 64/(D/8) token rows.  Lanes holding
// the same token ("row group") reduce their partial dot products with DPP;
// every row group keeps its own running (max, sum, acc) so the hot loop has
// no cross-row traffic; row groups are merged once per segment.  Scores are
// kept in log2 units (scale * log2 e folded in), so exp is one v_exp_f32.
#pragma once

#include "pa_internal.h"
#include "append.h"
#include "work_split.h"

#include <type_traits>

namespace pa {
namespace valu {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.693147180559945309f;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LANES (4, 8 or 16) lanes; every lane of the
// group receives the total.  quad_perm(1,0,3,2), quad_perm(2,3,0,1),
// row_half_mirror, row_mirror.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  if constexpr (LANES >= 8) x += dpp<0x141>(x);
  if constexpr (LANES >= 16) x += dpp<0x140>(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;   // v_cvt_f16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// Raw buffer resource over [base, base + bytes).  A load at an offset at or
// past `bytes` returns zero without touching memory, which is how prefetches
// past the last block are made free.  Word 3 = 0x00020000: raw 32-bit data
// format, no swizzle, no thread-id offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// K/V rows: each load instruction covers whole token rows (every 128-byte
// line it touches is read in full).  NT: the rows are not read again in this
// launch, so the loads carry the non-temporal cache policy; measured on
// llama2_7b this took the kernel from 353 to 320 us (the lines no longer
// compete for the caches).  Without NT (the shared-prefix launch, whose
// prefix work re-reads shared blocks from cache alongside) they use the
// default policy.
template <bool NT>
__device__ __forceinline__ void buffer_load(uint4& dst, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  u32x4 v = NT ? __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2)
               : __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  dst = make_uint4(v[0], v[1], v[2], v[3]);
}
template <bool NT>
__device__ __forceinline__ void buffer_load(uint2& dst, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  u32x2 v = NT ? __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2)
               : __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  dst = make_uint2(v[0], v[1]);
}
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

template <bool I8>
struct KvChunk;
template <>
struct KvChunk<false> { using T = uint4; static constexpr int kBytes = 16; };
template <>
struct KvChunk<true> { using T = uint2; static constexpr int kBytes = 8; };

// 8 elements of a chunk as fp32.
__device__ __forceinline__ void to_f32(const uint4& c, float (&f)[8]) {
  h8 v = __builtin_bit_cast(h8, c);
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (float)v[e];
}
__device__ __forceinline__ void i8_to_f32(const uint2& c, float (&f)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = (float)(int)(int8_t)(c.x >> (8 * e));
#pragma unroll
  for (int e = 0; e < 4; ++e) f[4 + e] = (float)(int)(int8_t)(c.y >> (8 * e));
}
// Eight OCP E4M3 codes, exact (v_cvt_pk_f32_fp8, two codes per call).
__device__ __forceinline__ void f8_to_f32(const uint2& c, float (&f)[8]) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, true);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, false);
  const auto e = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, true);
  f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
  f[4] = d[0]; f[5] = d[1]; f[6] = e[0]; f[7] = e[1];
}
// Values of one chunk of K/V elements in format KV.
template <int KV>
__device__ __forceinline__ void kv_to_f32(const typename KvChunk<KV != kKvF16>::T& c,
                                          float (&f)[8]) {
  if constexpr (KV == kKvI8) i8_to_f32(c, f);
  else if constexpr (KV == kKvF8) f8_to_f32(c, f);
  else to_f32(c, f);
}

template <int D, int G, int KV, bool NT>
__device__ __forceinline__ void valu_body(const DecodeParams& p, const int wg) {
  constexpr bool I8 = KV != kKvF16;          // 8-bit codes with per-token scales
  constexpr int LPR = D / 8;                 // lanes per token row
  constexpr int RPW = 64 / LPR;              // token rows per wave load
  constexpr int NL = kBlockTokens / RPW;     // wave loads per block
  using Chunk = typename KvChunk<I8>::T;
  constexpr int ESZ = I8 ? 1 : 2;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wpg = blockDim.x >> 6;           // kv heads per workgroup
  const int r = lane / LPR, c = lane % LPR;
  const int Hq = p.q_heads, Hkv = p.kv_heads;

  // Append mode: the workgroups past the partition work write the newest
  // tokens and their records (append.h).
  if (p.k_new != nullptr && wg >= p.main_groups) {
    const long long pair = (long long)(wg - p.main_groups) * wpg + w;
    if (pair < (long long)p.batch * Hkv) append_token<D, G, KV>(p, (int)pair);
    return;
  }

  // Workgroup item: a balanced chunk of blocks, a (partition, sequence) or a
  // sequence, with a head group (locate_work).  A chunk may cross sequence
  // boundaries; each sequence it reaches is one segment with its own record.
  const int groups = Hkv / wpg;
  Segment sg = locate_work(p, groups, wg);
  const int g = sg.grp * wpg + w;
  const int h0 = g * G;
  if (!p.direct && wg == 0 && tid == 0)
    p.header[0] = (long long)p.batch * Hkv >= p.target_waves ? 1 : 0;
  if (sg.b < 0) return;                      // no work for this workgroup

  // Addressing: a block's rows for kv head g start at a wave-uniform base
  // (scalar registers); each lane adds a fixed 32-bit offset per load.
  const uint32_t blk_bytes = (uint32_t)kBlockTokens * Hkv * D * ESZ;
  uint32_t lane_off[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i)
    lane_off[i] = ((uint32_t)(r + RPW * i) * Hkv * D + (uint32_t)g * D + (uint32_t)c * 8) * ESZ;
  uint32_t scale_off[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) scale_off[i] = (uint32_t)g * kBlockTokens + r + RPW * i;   // [NB, Hkv, 16]
  const char* kbase = static_cast<const char*>(p.k_pool);
  const char* vbase = static_cast<const char*>(p.v_pool);
  const uint32_t scale_blk_bytes = (uint32_t)kBlockTokens * Hkv * sizeof(float);

  do {                                       // segments of the item
  note_record_count(p, sg, w == 0 && lane == 0);
  // The segment's fields are wave-uniform; saying so keeps every value
  // derived from them (lengths, block counts, buffer resources) in scalar
  // registers across the segment loop.
  const int b = __builtin_amdgcn_readfirstlane(sg.b);
  const int ridx = __builtin_amdgcn_readfirstlane(sg.rec);
  const int seg_j0 = __builtin_amdgcn_readfirstlane(sg.j0);
  const int seg_blocks = __builtin_amdgcn_readfirstlane(sg.nblk);
  const int seg_len = __builtin_amdgcn_readfirstlane(sg.len);
  const int t_begin = seg_j0 * kBlockTokens;
  const int j0 = min(seg_j0, p.max_blocks - 1);
  const int32_t* bt_row =
      p.block_table + (size_t)b * p.bt_stride + p.token_offset / kBlockTokens;

  // Start-up loads, independent of each other: the length (unless the
  // search already read it), the first 64 block ids of the segment (clamped
  // to the table row) and Q.
  const int L = seg_len >= 0 ? seg_len : seq_len(p, b);
  const int row_left = p.max_blocks - j0;
  // Block ids c0 .. c0+63 of the segment, one per lane, through a buffer
  // resource bounded to the segment's slice of the table row: ids past the
  // slice read as 0 with no branch, so the load stays asynchronous.
  const __amdgpu_buffer_rsrc_t rids =
      make_rsrc(bt_row + j0, (uint32_t)max(min(seg_blocks, row_left), 0) * 4u);
  auto load_ids = [&](int c0) {
    return (int)__builtin_amdgcn_raw_buffer_load_b32(rids, (uint32_t)(c0 + lane) * 4u, 0, 0);
  };
  int ids = load_ids(0);
  // Query slice of every head in the group: elements c*8 .. c*8+7.
  uint4 qraw[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
    qraw[hh] = *reinterpret_cast<const uint4*>(p.q + ((size_t)b * Hq + h0 + hh) * D + c * 8);

  // Empty or broken sequences only reach here as single-segment items
  // (direct mode or partition items); chunks skip them.
  if (L < 0 || L > p.max_context_len) {      // broken metadata: NaN rows
    if (ridx == 0 && p.direct) {
      for (int i = lane; i < G * D; i += 64) {
        const size_t row = (size_t)b * Hq + h0 + i / D;
        p.out[row * D + i % D] = 0x7E00;
        if (i % D == 0 && p.lse) p.lse[row] = __builtin_nanf("");
      }
    }
    return;
  }
  if (t_begin >= L) {                        // empty item (L == 0: zero row)
    if (p.direct && ridx == 0) {
      for (int i = lane; i < G * D; i += 64) {
        const size_t row = (size_t)b * Hq + h0 + i / D;
        p.out[row * D + i % D] = 0;
        if (i % D == 0 && p.lse) p.lse[row] = kNegInf;
      }
    }
    return;
  }
  const int ntok = min(t_begin + seg_blocks * kBlockTokens, L) - t_begin;
  const int nfull = ntok / kBlockTokens;
  const int tail = ntok - nfull * kBlockTokens;

  float qf[I8 ? G : 1][8];
  if constexpr (I8) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) to_f32(qraw[hh], qf[hh]);
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = kNegInf;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
  }
  bool bad_blk = false;

  struct Regs {
    Chunk k[NL];
    Chunk v[NL];
    float ks[NL];
    float vs[NL];
  };

  // Every K load of a block, then every V load (V arrives while the scores
  // are computed).  real == false: a prefetch past the end; its resource is
  // empty, so the loads return zeros without touching memory.  Rows at or
  // past `rows` (the partial last block) are read at an offset past the
  // resource's end, which likewise returns zeros without a memory access:
  // they are masked out anyway, and on short sequences they are a few
  // percent of the bytes.
  auto load_block = [&](int blk, bool real, int rows, Regs& R) {
    if ((unsigned)blk >= (unsigned)p.num_blocks) {
      if (real) bad_blk = true;              // the record becomes NaN
      real = false;
      blk = 0;
    }
    const uint32_t nbytes = real ? blk_bytes : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (size_t)blk * blk_bytes, nbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (size_t)blk * blk_bytes, nbytes);
    uint32_t off[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) off[i] = (r + RPW * i < rows) ? lane_off[i] : blk_bytes;
#pragma unroll
    for (int i = 0; i < NL; ++i) buffer_load<NT>(R.k[i], rk, off[i]);
#pragma unroll
    for (int i = 0; i < NL; ++i) buffer_load<NT>(R.v[i], rv, off[i]);
    if constexpr (I8) {
      const uint32_t sbytes = real ? scale_blk_bytes : 0u;
      const size_t sblk = (size_t)blk * kBlockTokens * Hkv;
      const __amdgpu_buffer_rsrc_t rks = make_rsrc(p.k_scale + sblk, sbytes);
      const __amdgpu_buffer_rsrc_t rvs = make_rsrc(p.v_scale + sblk, sbytes);
#pragma unroll
      for (int i = 0; i < NL; ++i) R.ks[i] = buffer_load_f32(rks, scale_off[i] * 4u);
#pragma unroll
      for (int i = 0; i < NL; ++i) R.vs[i] = buffer_load_f32(rvs, scale_off[i] * 4u);
    }
  };

  // Online-softmax update of every head of the group with one block.  TAIL:
  // rows at or past `valid` are masked out (they may hold anything, NaN
  // included).
  auto process_block = [&](auto tail_tag, const Regs& R, int valid) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    float s[G][NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float kf[I8 ? 8 : 1];
      if constexpr (I8) kv_to_f32<KV>(R.k[i], kf);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float part_dot = 0.f;
        if constexpr (I8) {
#pragma unroll
          for (int e = 0; e < 8; ++e) part_dot = fmaf(qf[hh][e], kf[e], part_dot);
        } else {
          const uint32_t* qw = reinterpret_cast<const uint32_t*>(&qraw[hh]);
          const uint32_t* kw = reinterpret_cast<const uint32_t*>(&R.k[i]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            part_dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, qw[e]),
                                              __builtin_bit_cast(h2, kw[e]), part_dot, false);
        }
        s[hh][i] = part_dot;
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float sc = group_sum<LPR>(s[hh][i]) * p.scale_log2;
        if constexpr (I8) sc *= R.ks[i];
        if constexpr (TAIL) {
          if (r + RPW * i >= valid) sc = kNegInf;
        }
        s[hh][i] = sc;
      }
    }
    // Rescale by the new running max; the scores become probabilities.
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float mb = s[hh][0];
#pragma unroll
      for (int i = 1; i < NL; ++i) mb = fmaxf(mb, s[hh][i]);
      const float m_new = fmaxf(m[hh], mb);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m[hh] - m_use);
      l[hh] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        s[hh][i] = fast_exp2(s[hh][i] - m_use);
        l[hh] += s[hh][i];
      }
      m[hh] = m_new;
    }
    // V rows one load at a time (each converted once for all heads of the
    // group), so only one load's values are live as fp32.
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float vf[8];
      kv_to_f32<KV>(R.v[i], vf);
      float vsc = R.vs[i];
      if constexpr (TAIL) {
        if (r + RPW * i >= valid) {   // masked row: value and its scale may be NaN
#pragma unroll
          for (int e = 0; e < 8; ++e) vf[e] = 0.f;
          vsc = 0.f;
        }
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float pv = I8 ? s[hh][i] * vsc : s[hh][i];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(pv, vf[e], acc[hh][e]);
      }
    }
  };

  // Record of the segment: merge the RPW row groups, then store.
  auto finalize = [&]() {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float M = m[hh];
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
      const float f = fast_exp2(m[hh] - ((M == kNegInf) ? 0.f : M));
      float den = l[hh] * f;
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) den += __shfl_xor(den, off);
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = acc[hh][e] * f;
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) x += __shfl_xor(x, off);
        o[e] = x;
      }
      if (bad_blk) M = den = __builtin_nanf("");
      if (r == 0) {                          // lanes c = 0 .. LPR-1 hold dims c*8 .. c*8+7
        const size_t row = (size_t)b * Hq + h0 + hh;
        if (p.direct) {
          const float inv = 1.0f / den;
          uint4 pk;
          uint32_t* pw = reinterpret_cast<uint32_t*>(&pk);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pw[e] = (uint32_t)f32_to_f16_bits(o[2 * e] * inv) |
                    ((uint32_t)f32_to_f16_bits(o[2 * e + 1] * inv) << 16);
          if (bad_blk) pk = make_uint4(0x7E007E00u, 0x7E007E00u, 0x7E007E00u, 0x7E007E00u);
          *reinterpret_cast<uint4*>(p.out + row * D + c * 8) = pk;
          if (c == 0 && p.lse) p.lse[row] = (M + log2f(den)) * kLn2;
        } else {
          // o / l in fp16 (a convex combination of V rows, so within V's
          // range); (m, l) stay fp32.
          const size_t rec = (size_t)ridx * ((size_t)p.batch * Hq) + row;   // record-major
          const float inv = 1.0f / den;
          uint4 pk;
          uint32_t* pw = reinterpret_cast<uint32_t*>(&pk);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pw[e] = (uint32_t)f32_to_f16_bits(o[2 * e] * inv) |
                    ((uint32_t)f32_to_f16_bits(o[2 * e + 1] * inv) << 16);
          if (bad_blk) pk = make_uint4(0x7E007E00u, 0x7E007E00u, 0x7E007E00u, 0x7E007E00u);
          *reinterpret_cast<uint4*>(p.part_o + rec * D + c * 8) = pk;
          if (c == 0) p.part_ml[rec] = make_float2(M, den);
        }
      }
    }
  };

  // Blocks of the segment, streamed in order.  Block ids come one per lane from
  // `ids`, a 64-block chunk; the following chunk is fetched into `ids_next`
  // a whole chunk ahead and moved over just before its first block is
  // issued, so no issue reads a register whose load may still be pending.
  // Two register sets alternate, so one block is in flight while the other
  // is reduced; block j always lands in R[j % 2].  The partial last block
  // (only in a sequence's last segment) is fetched through the same pipeline as
  // block nfull and reduced after the loop; later prefetches read nothing
  // (empty resource) and, with two sets, never land on the tail's set.
  // Every branch is wave-uniform and no load sits inside one, so the waits
  // stay exact.
  constexpr int NBUF = 2;
  const int nreal = nfull + (tail > 0 ? 1 : 0);
  int ids_next = load_ids(64);
  int next_chunk = 1;                        // chunk held in `ids_next`
  auto issue = [&](int k, Regs& R) {
    const bool real = k < nreal;
    load_block(__builtin_amdgcn_readlane(ids, real ? (k & 63) : 0), real,
               k == nfull ? tail : kBlockTokens, R);
  };
  auto done = [&](int k) {                   // block k reduced; k + NBUF is issued next
    if (((k + NBUF) & 63) == 0 && k + NBUF < nreal) {
      ids = ids_next;
      ++next_chunk;
      ids_next = load_ids(next_chunk * 64);
    }
  };
  std::integral_constant<bool, false> full;
  Regs R[NBUF];
  issue(0, R[0]);
  for (int k = 0; k < nfull; k += NBUF) {
#pragma unroll
    for (int s = 0; s < NBUF; ++s) {
      issue(k + s + 1, R[(s + 1) % NBUF]);
      __builtin_amdgcn_sched_barrier(0);
      if (s == 0 || k + s < nfull) {
        process_block(full, R[s], kBlockTokens);
        done(k + s);
      }
    }
  }
  if (tail > 0) {
    std::integral_constant<bool, true> last;
    if (nfull & 1)
      process_block(last, R[1], tail);
    else
      process_block(last, R[0], tail);
  }
  finalize();
  } while (next_segment(p, sg));
}

}  // namespace valu
}  // namespace pa
