// Paged-attention decode, split-K partition kernel for grouped query heads
// (G = q_heads / kv_heads in {4, 8, 16}) on gfx950 matrix cores.
//
// With G query heads sharing one kv head, each K/V row is used G times, so
// the dot products and the V accumulation form real tiles:
//   S^T[t][h] = sum_d K[t][d] Q[h][d]     16 tokens x 16 heads, k = head_dim
//   O^T[d][h] += sum_t V[t][d] P[h][t]    16 dims  x 16 heads, k = 16 tokens
// Heads are padded to 16 (rows h >= G hold zeros and are never stored).
// The first product takes K straight from the global loads as the A operand
// of v_mfma_f32_16x16x32_f16 (a lane holds 8 elements of one token row).  In
// the result every lane owns one head (lane % 16) and four tokens, so the
// online softmax needs only one cross-row max per block.  The second product
// needs V with tokens along the contraction; V is staged in LDS in its
// natural [token][dim] order and read back transposed with ds_read_b64_tr_b16,
// and the probabilities already sit in the B-operand layout of
// v_mfma_f32_16x16x16_f16.  O^T keeps the head on lane % 16, so the
// per-head rescale by the running-max correction is a per-lane multiply.
//
// int8 caches: codes are converted exactly to fp16 (0x6400 | (x ^ 0x80) is
// 1152 + x; subtracting 1152 in packed fp16 leaves x), the per-token K scale
// is applied to the score and the V scale to the probability.  FP8 (OCP
// E4M3) caches: every E4M3 value is exact in fp16, two codes per
// v_cvt_scalef32_pk_f16_fp8 (scale 1); the scales are applied as for int8.
// The probability times the V scale enters the PV product in fp16, relative
// to a power of two 2^vexp kept per segment (see vexp below), so small
// scales do not push it into fp16's subnormal range; finalize multiplies
// the result back by 2^vexp, exactly.
//
// Method and readings are those of the VALU kernel (zskr.cn ATB
// PagedAttention article, section "PagedAttention 的 Attention 计算修改",
// with the running max updated before the exponent, -inf start, a scale,
// fp32 accumulation, per-head output and masked tail slots; the page table
// staged on chip once per workgroup, section "踩坑一"; query heads grouped on
// one K/V head, discosf.com article, section "二、优化方向").
#pragma once

#include "pa_internal.h"
#include "append.h"
#include "work_split.h"

#include <type_traits>

namespace pa {
namespace mfma {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;   // at most eight waves (kv heads) per workgroup
// Block ids of a segment staged in LDS per workgroup, refilled kIdCap at a time.
constexpr int kIdCap = 1024;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.693147180559945309f;
#ifndef PA_V_ROW_PAD
#define PA_V_ROW_PAD 16
#endif
constexpr int kRowPad = PA_V_ROW_PAD;   // bytes of padding per LDS row of the V tile
// 1: the V tile's rows are unpadded and the 16-byte chunks of row r sit at
// chunk c ^ swz(r) (see v_swizzle); 0: rows padded by kRowPad bytes.
#ifndef PA_V_SWIZZLE
#define PA_V_SWIZZLE 1
#endif
// Register sets the block loads rotate through (NBUF - 1 blocks in flight
// while one is reduced).
#ifndef PA_MFMA_NBUF_I8
#define PA_MFMA_NBUF_I8 3
#endif
#ifndef PA_MFMA_NBUF_F16
#define PA_MFMA_NBUF_F16 2
#endif
#ifndef PA_MFMA_WAVES_PER_EU
#define PA_MFMA_WAVES_PER_EU 3
#endif
#ifndef PA_MFMA_WHOLE_LINE
#define PA_MFMA_WHOLE_LINE 1
#endif
#ifndef PA_MFMA_KV_NT
#define PA_MFMA_KV_NT 1
#endif
#ifndef PA_MFMA_K_EXACT
#define PA_MFMA_K_EXACT 0
#endif
// The running max is only moved (and the accumulators rescaled) when a block
// beats it by more than this many log2 units; softmax is invariant to the
// reference point, and probabilities stay <= 2^8, well inside fp16.
constexpr float kRescaleSlack = 8.0f;
// 8-bit caches: the V scales of a block enter the fp16 probabilities as
// scale * 2^-vexp.  vexp follows the largest scale exponent e of the blocks
// (floor(log2)), moving only when a block leaves [vexp - kVexpDown,
// vexp + kVexpUp]; a move multiplies the accumulators by a power of two,
// exactly.  With p <= 2^8 the fp16 operand stays below 2^(8 + kVexpUp + 1)
// = 2^15 (finite); a token whose scale is within 2^-kVexpDown of vexp and
// whose probability is at least 2^-6 stays in fp16's normal range.
constexpr int kVexpUp = 6;
constexpr int kVexpDown = 8;
constexpr int kLongContext = 32768;   // tokens; see waves_per_group

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the four lane groups l, l^16, l^32, l^48 (the lanes that
// share a query slot).  gfx950's permlane swaps trade row halves between two
// registers on the VALU, without the LDS round trip of a lane shuffle: with
// both operands equal to x, the swapped pair holds x[l] and x[l ^ 32] (then
// x[l ^ 16]) in every lane, each pair ordered low lane first, so both lanes
// of a pair compute the same value.
__device__ __forceinline__ float group_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float group_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// K/V loads; NT: the non-temporal cache policy (whole lines read once).
template <bool NT>
__device__ __forceinline__ uint4 buffer_load16_kv(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  u32x4 v = NT ? __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2)
               : __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Lane l ^ 8 within each row of 16 lanes (DPP row rotation by 8).
__device__ __forceinline__ uint32_t swap8(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);
}

// Four int8 codes -> four exact fp16 values.
__device__ __forceinline__ void i8x4_to_h4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = w ^ 0x80808080u;                          // x + 128 as unsigned bytes
  lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);     // halves 0x64xx: 1024 + byte
  hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const h2 off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, lo) + off);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, hi) + off);
}

// Four int8 codes -> four fp16 values 1152 + x (exact; the bias is removed
// from the dot product as 1152 * sum(q) instead of per element).
__device__ __forceinline__ void i8x4_to_h4_biased(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = w ^ 0x80808080u;
  lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
}

__device__ __forceinline__ void i8x16_to_h16_biased(const uint4& c, uint4& first, uint4& second) {
  i8x4_to_h4_biased(c.x, first.x, first.y);
  i8x4_to_h4_biased(c.y, first.z, first.w);
  i8x4_to_h4_biased(c.z, second.x, second.y);
  i8x4_to_h4_biased(c.w, second.z, second.w);
}

// 16 int8 codes -> 16 fp16 (two 8-element halves).
__device__ __forceinline__ void i8x16_to_h16(const uint4& c, uint4& first, uint4& second) {
  i8x4_to_h4(c.x, first.x, first.y);
  i8x4_to_h4(c.y, first.z, first.w);
  i8x4_to_h4(c.z, second.x, second.y);
  i8x4_to_h4(c.w, second.z, second.w);
}

// Four E4M3 codes -> four fp16 (codes 0, 1 in lo; 2, 3 in hi).
__device__ __forceinline__ void f8x4_to_h4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, true));
}

__device__ __forceinline__ void f8x16_to_h16(const uint4& c, uint4& first, uint4& second) {
  f8x4_to_h4(c.x, first.x, first.y);
  f8x4_to_h4(c.y, first.z, first.w);
  f8x4_to_h4(c.z, second.x, second.y);
  f8x4_to_h4(c.w, second.z, second.w);
}

// Which bytes of a block each lane loads, and which head-dim elements it then
// feeds to the QK product: in the operand layout lane (li, g) holds bytes
// 64 ld + 16 g .. + 15 of its head's row in token li, as the A operand
// wants.  The loads themselves read whole 128-byte lines (see load_row), so
// each line is consumed by one instruction and can carry the non-temporal
// cache policy; with the default policy the half-line layout and the
// whole-line one measured within 2 %.
template <int D, bool I8>
struct Geometry {
  static constexpr int kEsz = I8 ? 1 : 2;
  // 16-byte global loads per lane per block for K (and again for V).
  static constexpr int kLoads = D * kEsz / 64;
  // QK MFMA steps (8 elements of k per lane each).
  static constexpr int kSteps = D / 32;
  // Head-dim element held by lane group g, element j of QK step kk.
  static __device__ __forceinline__ int dim(int kk, int g, int j) {
    if constexpr (I8) return 64 * (kk / 2) + 16 * g + 8 * (kk % 2) + j;
    else return 32 * kk + 8 * g + j;
  }
  // Loads come in pairs over one 128-byte line of every token row
  // (whole-line mode, when a head's row spans at least one line): load 2m
  // reads rows 0..7 and load 2m+1 rows 8..15, each row's whole line, so no
  // line is left half read.  Lane (li, lg) of load 2m reads row li & 7 at
  // chunk lg (li < 8) or lg + 4 (li >= 8); of load 2m+1, row 8 + (li & 7) at
  // chunk lg (li >= 8) or lg + 4 (li < 8) (16-byte chunks of the line).  So
  // lane (li, lg) already holds chunk lg of its own row li in one of the
  // two, and chunk lg + 4 of row li sits in lane (li ^ 8, lg) of the other:
  // one select and one DPP row rotation by 8 restore the operand layout
  // below (kswap).  Otherwise (a 64-byte row) load ld reads bytes
  // 64 ld + 16 lg of row li.
  static constexpr bool kWholeLine = kLoads >= 2 && PA_MFMA_WHOLE_LINE;
  static __device__ __forceinline__ int load_row(int ld, int lane) {
    const int li = lane & 15;
    if constexpr (kWholeLine) return (ld & 1) ? 8 + (li & 7) : (li & 7);
    else return li;
  }
  static __device__ __forceinline__ int load_col(int ld, int lane) {
    const int li = lane & 15, lg = lane >> 4;
    if constexpr (kWholeLine) {
      const bool low = li < 8;
      const int chunk = lg + (((ld & 1) ? low : !low) ? 4 : 0);
      return 128 * (ld >> 1) + 16 * chunk;
    } else {
      return 64 * ld + 16 * lg;
    }
  }
  static constexpr int kRowBytes = D * 2 + (PA_V_SWIZZLE ? 0 : kRowPad);   // LDS row of the V tile
  // 16-byte chunks per row of the fp16 V tile.
  static constexpr int kChunks = D * 2 / 16;
  // Chunk c of V-tile row r is stored at chunk c ^ v_swizzle(r).  A block's
  // V goes in as 16-byte writes (whole-line loads: the 16 lanes of one lane
  // group write rows 0..7 at chunks c and c + 4 (fp16) or c and c + 8
  // (int8, two writes per lane)) and comes out through ds_read_b64_tr_b16
  // (lanes 0..31 read rows 0..7, 32 bytes each, at the same chunk pair).
  // The table below puts the 8 rows' chunk pairs on 8 different 32-byte bank
  // groups for the reads, and the 16 chunks of a lane group's write on 16
  // different 16-byte bank groups, both with 64 four-byte banks served 16
  // (writes) or 32 (reads) lanes at a time and with 32 banks served 8 or 16
  // lanes at a time: for row r & 7 = 0..7 it is 0, 2, 12, 14, 9, 11, 5, 7
  // (an odd low bit moves the 16-byte chunks a lane group writes to the
  // other half of the banks), taken modulo the row's chunks.  The padded
  // layout it replaces had two-way conflicts on every transposed read.
  static __device__ __forceinline__ int v_swizzle(int row) {
    if constexpr (!PA_V_SWIZZLE) return 0;
    const int t = 2 * (row & 3) + ((row >> 2) & 1);
    const int beta = (t & 1) ^ ((t >> 2) & 1);
    return (t + 8 * beta) & (kChunks - 1);
  }
  // LDS byte address of 16-byte chunk `chunk` of V-tile row `row`.
  static __device__ __forceinline__ uint32_t v_addr(int row, int chunk) {
    return (uint32_t)row * kRowBytes + (uint32_t)((chunk ^ v_swizzle(row)) * 16);
  }
};

// Scale of token 4 lg + i from a register holding, at row position p, the
// scale of token (p + 4 lg) % 16: broadcast of row position i (DPP
// row_newbcast, no memory access).
__device__ __forceinline__ float scale_of(float x, int i) {
  switch (i) {
    case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150, 0xF, 0xF, false));
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x151, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x152, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x153, 0xF, 0xF, false));
  }
}

// Three waves per SIMD (<= 168 registers) with two (fp16) or three (int8)
// register sets of block loads; deeper rotation at two waves per SIMD and
// four waves per SIMD with fewer sets both measured slower.
//
// Work split: a workgroup holds `wpg` waves (1, 2, 4 or 8) for wpg consecutive
// kv heads of one work item (work_split.h); each wave streams its own head's
// blocks of the item and writes its own record per sequence.  The waves of a
// workgroup thus read neighbouring slices of the same token rows at the same
// time, and a wave's start-up (lengths, block ids, Q) is paid once per
// segment.
template <int D, int G, int KV, bool PREFIX>
__device__ __forceinline__ void mfma_body(const DecodeParams& p, const int wg) {
  constexpr bool I8 = KV != kKvF16;          // 8-bit codes with per-token scales
  using Geo = Geometry<D, I8>;
  constexpr int NLD = Geo::kLoads;
  constexpr int NKK = Geo::kSteps;
  constexpr bool kLineNT = Geo::kWholeLine && PA_MFMA_KV_NT;
  constexpr int NT = D / 16;                 // O^T tiles of 16 dims
  constexpr int ESZ = I8 ? 1 : 2;
  constexpr int TILE = kBlockTokens * Geo::kRowBytes;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wpg = blockDim.x >> 6;           // kv heads per workgroup
  const int lg = lane >> 4;       // lane group 0..3
  const int li = lane & 15;       // index in group: token row for loads, head for softmax
  const int Hq = p.q_heads, Hkv = p.kv_heads;

  // Append mode: the workgroups past the partition work write the newest
  // tokens and their records (append.h).
  if constexpr (!PREFIX) {
    if (p.k_new != nullptr && wg >= p.main_groups) {
      const long long pair = (long long)(wg - p.main_groups) * wpg + w;
      if (pair < (long long)p.batch * Hkv) append_token<D, G, KV>(p, (int)pair);
      return;
    }
  }

  // Workgroup item: a balanced chunk of blocks, a (partition, sequence) or a
  // sequence, with a head group (locate_work); a chunk may cross sequence
  // boundaries, and each sequence it reaches is one segment with its own
  // record.  Shared prefix: item = (query tile, partition, head group), head
  // groups fastest; the stream is table row 0 over the prefix.
  const int groups = Hkv / wpg;
  Segment sg;
  int tile = 0;
  int g_prefix = 0;
  if constexpr (PREFIX) {
    if (p.prefix_tile_waves) {
      // item = (tile group, partition, kv head), kv heads fastest; wave w
      // takes query tile tile_group * wpg + w (a tile past the last one has
      // only padding slots and stores nothing)
      const int n_ph = p.n_part * Hkv;
      tile = (wg / n_ph) * wpg + w;
      const int part = (wg % n_ph) / Hkv;
      g_prefix = wg % Hkv;
      sg = Segment{0, -1, part * (p.partition_size / kBlockTokens),
                   p.partition_size / kBlockTokens, part, 0, 0, 0, -1, 0, 0};
    } else {
      const int n_rg = p.n_part * groups;
      tile = wg / n_rg;
      const int part = (wg % n_rg) / groups;
      sg = Segment{0, -1, part * (p.partition_size / kBlockTokens),
                   p.partition_size / kBlockTokens, part, (int)(wg % groups), 0, 0, -1, 0, 0};
      g_prefix = sg.grp * wpg + w;
    }
  } else {
    sg = locate_work(p, groups, wg);
    if (!p.direct && wg == 0 && tid == 0)
      p.header[0] = (long long)p.batch * Hkv >= p.target_waves ? 1 : 0;
    if (sg.b < 0) return;                    // no work for this workgroup
  }
  const int g = PREFIX ? g_prefix : sg.grp * wpg + w;
  const int h0 = g * G;

  char* s_tile = smem + w * TILE;            // this wave's V tile
  // Block ids of the segment, shared by the workgroup (all its waves stream
  // the same blocks, so every step below is taken by all of them together).
  int32_t* s_ids = reinterpret_cast<int32_t*>(smem + wpg * TILE);

  const uint32_t row_bytes = (uint32_t)Hkv * D * ESZ;          // one token row, all heads
  const uint32_t blk_bytes = (uint32_t)kBlockTokens * row_bytes;
  // Offsets of this lane's loads within a block, and their V tile targets.
  uint32_t ld_off[NLD];
  // V tile address of the load's (first) 16 fp16 bytes; an 8-bit load's
  // second 16 bytes (chunk + 1 of an even chunk) sit at that address ^ 16.
  uint32_t ld_lds[NLD];
  int ld_row[NLD];
#pragma unroll
  for (int ld = 0; ld < NLD; ++ld) {
    ld_row[ld] = Geo::load_row(ld, lane);
    const int col = Geo::load_col(ld, lane);
    ld_off[ld] = (uint32_t)ld_row[ld] * row_bytes + (uint32_t)g * D * ESZ + (uint32_t)col;
    const int chunk = (col / ESZ) * 2 / 16;          // 16-byte chunk of the fp16 row
    ld_lds[ld] = Geo::v_addr(ld_row[ld], chunk);
  }
  const char* kbase = static_cast<const char*>(p.k_pool);
  const char* vbase = static_cast<const char*>(p.v_pool);
  const uint32_t scale_blk_bytes = (uint32_t)kBlockTokens * Hkv * sizeof(float);

  // LDS addresses of this lane's transposed V reads: for tile n, group lg
  // reads token row 4*lg + li/4 at dims 16*n + 4*(li%4) (8 bytes), i.e.
  // chunk 2n + (li%4)/2, byte 8*(li%2) of it.  Swizzled, that chunk sits at
  // (2n + (li%4)/2) ^ swz = 2 (n ^ (x >> 1)) + (x & 1) with x = swz ^ ((li%4)/2);
  // the rows start at multiples of the 256- or 128-byte row, so tile n's
  // address is tr_base ^ (32 n).
  const uint32_t tr_base = [&] {
    const int row = 4 * lg + li / 4;
    if constexpr (PA_V_SWIZZLE) {
      const int x = Geo::v_swizzle(row) ^ ((li % 4) >> 1);
      return (uint32_t)row * Geo::kRowBytes + (uint32_t)(32 * (x >> 1) + 16 * (x & 1) + 8 * (li & 1));
    } else {
      return (uint32_t)row * Geo::kRowBytes + (uint32_t)(4 * (li % 4)) * 2;
    }
  }();

  do {                                       // segments of the item
  if constexpr (!PREFIX) note_record_count(p, sg, tid == 0);
  // The segment's fields are wave-uniform; saying so keeps every value
  // derived from them (lengths, block counts, buffer resources) in scalar
  // registers across the segment loop.
  const int b = __builtin_amdgcn_readfirstlane(sg.b);
  const int ridx = __builtin_amdgcn_readfirstlane(sg.rec);
  const int seg_j0 = __builtin_amdgcn_readfirstlane(sg.j0);
  const int seg_blocks = __builtin_amdgcn_readfirstlane(sg.nblk);
  const int seg_len = __builtin_amdgcn_readfirstlane(sg.len);
  // Row of q / out / records of query slot li, or -1 for a padding slot.
  int qrow = -1;
  if constexpr (PREFIX) {
    const int Gm = Hq / Hkv;
    const int qi = tile * 16 + li;
    if (qi < p.batch * Gm) qrow = (qi / Gm) * Hq + g * Gm + qi % Gm;
  } else {
    if (li < G) qrow = b * Hq + h0 + li;
  }

  const int t_begin = seg_j0 * kBlockTokens;
  const int j0 = min(seg_j0, p.max_blocks - 1);
  const int32_t* bt_row =
      p.block_table + (size_t)b * p.bt_stride + p.token_offset / kBlockTokens;

  // Start-up loads, independent of each other: the length (unless the
  // search already read it) and Q.
  const int L = PREFIX ? p.max_context_len
                       : seg_len >= 0 ? seg_len : seq_len(p, b);
  const int row_left = p.max_blocks - j0;
  // The segment's slice of the table row as a buffer resource: ids past the
  // slice read as 0 with no branch.
  const __amdgpu_buffer_rsrc_t rids =
      make_rsrc(bt_row + j0, (uint32_t)max(min(seg_blocks, row_left), 0) * 4u);

  // Q^T as the B operand of the QK product: lane holds Q[slot li][dim(kk, lg, j)].
  // Each step's 8 dims are consecutive (Geo::dim), so one 16-byte load each;
  // padding slots load row 0 and are zeroed.
  h8 qB[NKK];
  {
    const uint16_t* qsrc = p.q + (size_t)(qrow >= 0 ? qrow : 0) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      uint4 v = *reinterpret_cast<const uint4*>(qsrc + Geo::dim(kk, lg, 0));
      if (qrow < 0) v = make_uint4(0, 0, 0, 0);
      qB[kk] = __builtin_bit_cast(h8, v);
    }
  }

  // Empty or broken sequences only reach here as single-segment items
  // (direct mode or partition items); chunks skip them.
  if (L < 0 || L > p.max_context_len) {      // broken metadata: NaN rows
    if (ridx == 0 && p.direct && qrow >= 0) {
      const size_t row = (size_t)qrow;
      for (int d = lg; d < D; d += 4) p.out[row * D + d] = 0x7E00;
      if (lg == 0 && p.lse) p.lse[row] = __builtin_nanf("");
    }
    return;
  }
  if (t_begin >= L) {                        // empty item (L == 0: zero row)
    if (p.direct && ridx == 0 && qrow >= 0) {
      const size_t row = (size_t)qrow;
      for (int d = lg; d < D; d += 4) p.out[row * D + d] = 0;
      if (lg == 0 && p.lse) p.lse[row] = kNegInf;
    }
    return;
  }
  const int ntok = min(t_begin + seg_blocks * kBlockTokens, L) - t_begin;
  const int nfull = ntok / kBlockTokens;
  // (the shared prefix is whole blocks: its length is a multiple of 16)
  const int tail = PREFIX ? 0 : ntok - nfull * kBlockTokens;

  // Ids come from LDS in order, each read NBUF blocks before its block is
  // issued, so no block waits on a table read.
  auto fill_ids = [&](int base) {            // ids base .. base + kIdCap - 1
    __syncthreads();                         // the previous chunk is read
    for (int t = tid; t < kIdCap; t += blockDim.x)
      s_ids[t] = (int)__builtin_amdgcn_raw_buffer_load_b32(rids, (uint32_t)(base + t) * 4u, 0, 0);
    __syncthreads();
  };

  // int8: sum over head_dim of q for head li (removes the 1152 bias of K).
  float qbias = 0.f;
  if constexpr (KV == kKvI8 && !PA_MFMA_K_EXACT) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int j = 0; j < 8; ++j) qbias += (float)qB[kk][j];
    }
    qbias = group_sum(qbias);
    qbias *= 1152.0f;
  }

  f4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;   // reference max of head li (same in all four lane groups)
  float l_run = 0.f;       // this lane's share of the running sum (its tokens)
  int vexp = 0;            // 8-bit caches: V-scale exponent reference (wave-uniform)
  bool bad_blk = false;

  struct Regs {
    uint4 k[NLD];
    uint4 v[NLD];
    float ks;       // 8-bit: scale of token (li + 4 lg) % 16 (rotated; see scale_of)
    float vs;
  };

  // Loads of one block.  real == false: a prefetch past the end; its
  // resource is empty, so the loads return zeros without touching memory.
  // Rows at or past `rows` (the partial last block) are read at an offset
  // past the resource's end, which likewise returns zeros without a memory
  // access; they are masked out anyway.
  auto load_block = [&](int blk, bool real, int rows, Regs& R) {
    if ((unsigned)blk >= (unsigned)p.num_blocks) {
      if (real) bad_blk = true;              // the record becomes NaN
      real = false;
      blk = 0;
    }
    const uint32_t nbytes = real ? blk_bytes : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (size_t)blk * blk_bytes, nbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (size_t)blk * blk_bytes, nbytes);
    uint32_t off[NLD];
#pragma unroll
    for (int ld = 0; ld < NLD; ++ld) off[ld] = ld_row[ld] < rows ? ld_off[ld] : blk_bytes;
#pragma unroll
    for (int ld = 0; ld < NLD; ++ld) R.k[ld] = buffer_load16_kv<kLineNT>(rk, off[ld]);
#pragma unroll
    for (int ld = 0; ld < NLD; ++ld) R.v[ld] = buffer_load16_kv<kLineNT>(rv, off[ld]);
    if constexpr (I8) {
      // scales [NB, Hkv, 16] of kv head g: one float per lane, rotated by
      // 4 lg within each row of 16 lanes so that the four tokens 4 lg .. 4 lg+3
      // of this lane's softmax slots sit at row positions 0..3 (scale_of).
      // Four bytes per lane: a 16-byte load per lane of the same 64 bytes
      // costs the vector memory path four times the lane data.
      const uint32_t sbytes = real ? scale_blk_bytes : 0u;
      const size_t sblk = (size_t)blk * kBlockTokens * Hkv;
      const uint32_t soff = ((uint32_t)g * kBlockTokens + (uint32_t)((li + 4 * lg) & 15)) * 4u;
      R.ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           make_rsrc(p.k_scale + sblk, sbytes), soff, 0, 0));
      R.vs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           make_rsrc(p.v_scale + sblk, sbytes), soff, 0, 0));
    }
  };
  auto process_block = [&](auto tail_tag, const Regs& R, int valid) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    // K as fp16 A operands, one per QK step.
    // K in the operand layout: lane (li, lg) holds bytes 64 ld + 16 lg of
    // row li in kr[ld] (whole-line loads: a select and a swap, see Geometry).
    uint4 kr[NLD];
#pragma unroll
    for (int m = 0; m < NLD; m += (Geo::kWholeLine ? 2 : 1)) {
      if constexpr (Geo::kWholeLine) {
        const bool low = li < 8;
        const uint4 x = R.k[m], y = R.k[m + 1];
        const uint4 own = low ? x : y, other = low ? y : x;
        kr[m] = own;
        kr[m + 1] = make_uint4(swap8(other.x), swap8(other.y), swap8(other.z), swap8(other.w));
      } else {
        kr[m] = R.k[m];
      }
    }
    h8 kA[NKK];
    if constexpr (I8) {
#pragma unroll
      for (int ld = 0; ld < NLD; ++ld) {
        uint4 a, c;
        if constexpr (KV == kKvI8 && PA_MFMA_K_EXACT) i8x16_to_h16(kr[ld], a, c);
        else if constexpr (KV == kKvI8) i8x16_to_h16_biased(kr[ld], a, c);
        else f8x16_to_h16(kr[ld], a, c);
        kA[2 * ld] = __builtin_bit_cast(h8, a);
        kA[2 * ld + 1] = __builtin_bit_cast(h8, c);
      }
    } else {
#pragma unroll
      for (int ld = 0; ld < NLD; ++ld) kA[ld] = __builtin_bit_cast(h8, kr[ld]);
    }
    f4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      s = __builtin_amdgcn_mfma_f32_16x16x32_f16(kA[kk], qB[kk], s, 0, 0, 0);

    // V into this wave's LDS tile, natural [token][dim] order (fp16); a
    // tail row past `valid` may hold NaN and is zeroed.
#pragma unroll
    for (int ld = 0; ld < NLD; ++ld) {
      const bool zero_row = TAIL && ld_row[ld] >= valid;
      char* dst = s_tile + ld_lds[ld];
      if constexpr (I8) {
        uint4 a, c;
        if constexpr (KV == kKvI8) i8x16_to_h16(R.v[ld], a, c);
        else f8x16_to_h16(R.v[ld], a, c);
        if (zero_row) a = c = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(dst) = a;
        *reinterpret_cast<uint4*>(s_tile + (ld_lds[ld] ^ 16u)) = c;
      } else {
        uint4 a = R.v[ld];
        if (zero_row) a = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(dst) = a;
      }
    }

    // Online softmax of head li over tokens 4*lg + i.
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x;
      if constexpr (I8) x = (s[i] - qbias) * (p.scale_log2 * scale_of(R.ks, i));
      else x = s[i] * p.scale_log2;
      if constexpr (TAIL) {
        if (4 * lg + i >= valid) x = kNegInf;
      }
      sc[i] = x;
    }
    float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mb = group_max(mb);
    // Move the reference max only when some head of the wave outgrows it.
    if (__builtin_amdgcn_ballot_w64(mb > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, mb);
      const float alpha = fast_exp2(m_run - ((m_new == kNegInf) ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(sc[i] - m_use);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    float sv = 0.f;          // 8-bit: this lane's V scale times 2^-vexp
    if constexpr (I8) {
      // The lane holds the scale of token (li + 4 lg) % 16; tail tokens
      // (whose slots may hold NaN) count as 0.
      float vs = R.vs;
      if constexpr (TAIL) {
        if (((li + 4 * lg) & 15) >= valid) vs = 0.f;
      }
      // Largest scale of the block: every row of 16 lanes holds all 16.
      float vmax = vs;
      vmax = fmaxf(vmax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(vmax), 0xB1, 0xF, 0xF, false)));
      vmax = fmaxf(vmax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(vmax), 0x4E, 0xF, 0xF, false)));
      vmax = fmaxf(vmax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(vmax), 0x141, 0xF, 0xF, false)));
      vmax = fmaxf(vmax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(vmax), 0x140, 0xF, 0xF, false)));
      const int ebits = (__builtin_amdgcn_readfirstlane(__float_as_int(vmax)) >> 23) & 0xFF;
      // Zero (no valid token, or a block outside the pool) and non-finite
      // scales leave the reference where it is.
      if (ebits != 0 && ebits != 0xFF) {
        const int e = ebits - 127;
        if (e > vexp + kVexpUp || e < vexp - kVexpDown) {
          const float f = __builtin_ldexpf(1.0f, vexp - e);
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[n] *= f;
          vexp = e;
        }
      }
      sv = __builtin_ldexpf(vs, -vexp);
    }
    h4 pB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float pv = pr[i];
      if constexpr (I8) {
        float vsc = scale_of(sv, i);
        if constexpr (TAIL) {
          if (4 * lg + i >= valid) vsc = 0.f;
        }
        pv *= vsc;
      }
      pB[i] = (_Float16)pv;
    }

    // O^T += V^T P^T, V^T read transposed from LDS.  (The empty asm keeps
    // the per-tile address XORs inside the loop: hoisted, they would hold
    // NT registers for the whole segment.)
    uint32_t trb = tr_base;
    if constexpr (PA_V_SWIZZLE) asm volatile("" : "+v"(trb));
    typedef __attribute__((address_space(3))) s4 lds_s4;
    const __attribute__((address_space(3))) char* tile3 =
        (const __attribute__((address_space(3))) char*)(s_tile);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const uint32_t at = PA_V_SWIZZLE ? (trb ^ (uint32_t)(n * 32)) : trb + n * 32;
      s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(tile3 + at));
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4, a), pB, acc[n], 0,
                                                     0, 0);
    }
  };

  // Record of the segment: (m_run, l) and the normalised output.
  // Lane (lg, li) holds O[head li][dim 16n + 4lg + i].
  auto finalize = [&]() {
    float den = l_run;
    den = group_sum(den);
    // 1 / l, times 2^vexp for 8-bit caches (the V scales entered as
    // scale * 2^-vexp).
    const float inv_l = I8 ? __builtin_ldexpf(1.0f / den, vexp) : 1.0f / den;
    if (qrow >= 0) {
      const size_t row = (size_t)qrow;
      float M = m_run;
      if (bad_blk) M = den = __builtin_nanf("");
      if (p.direct) {
        const float inv = inv_l;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          uint2 o;
          o.x = (uint32_t)f32_to_f16_bits(acc[n][0] * inv) |
                ((uint32_t)f32_to_f16_bits(acc[n][1] * inv) << 16);
          o.y = (uint32_t)f32_to_f16_bits(acc[n][2] * inv) |
                ((uint32_t)f32_to_f16_bits(acc[n][3] * inv) << 16);
          if (bad_blk) o = make_uint2(0x7E007E00u, 0x7E007E00u);
          *reinterpret_cast<uint2*>(p.out + row * D + 16 * n + 4 * lg) = o;
        }
        if (lg == 0 && p.lse) p.lse[row] = (M + log2f(den)) * kLn2;
      } else {
        // o / l in fp16 (a convex combination of V rows, so within V's
        // range); (m, l) stay fp32.  Records are stored record-major (slot
        // ridx of every row together), so a wave's G rows are one run.
        const size_t rec = (size_t)ridx * ((size_t)p.batch * Hq) + row;
        const float inv = inv_l;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          uint2 o;
          o.x = (uint32_t)f32_to_f16_bits(acc[n][0] * inv) |
                ((uint32_t)f32_to_f16_bits(acc[n][1] * inv) << 16);
          o.y = (uint32_t)f32_to_f16_bits(acc[n][2] * inv) |
                ((uint32_t)f32_to_f16_bits(acc[n][3] * inv) << 16);
          if (bad_blk) o = make_uint2(0x7E007E00u, 0x7E007E00u);
          *reinterpret_cast<uint2*>(p.part_o + rec * D + 16 * n + 4 * lg) = o;
        }
        if (lg == 0) p.part_ml[rec] = make_float2(M, den);
      }
    }
  };

  // The segment's blocks: the partial last block (a sequence's last segment
  // only) first, then the full blocks in order.  Softmax does not depend on
  // the order, and loading the partial block with the first full ones
  // overlaps its memory latency with theirs instead of paying it again after
  // the full blocks drain.  Register sets rotate so that NBUF - 1 blocks are
  // in flight while one is reduced (int8 blocks are half the bytes, so they
  // go one deeper); the partial block's set is free again before the
  // rotation needs its last one.  Loads that have nothing to read (no
  // partial block, prefetches past the end) use an empty buffer resource
  // and fetch nothing, so every load is issued unconditionally.  Block ids:
  // each register set carries nid, the id of the next block it will
  // receive, read from LDS when its current block is issued.  Every branch
  // is wave-uniform (workgroup-uniform where it holds a barrier) and no
  // vector load sits inside one, so the waits stay exact.
  constexpr int NBUF = I8 ? PA_MFMA_NBUF_I8 : PA_MFMA_NBUF_F16;
  std::integral_constant<bool, false> full;
  // Id of the partial last block (read as 0 past the segment's slice).
  const int tail_id = (int)__builtin_amdgcn_raw_buffer_load_b32(rids, (uint32_t)nfull * 4u, 0, 0);
  fill_ids(0);                               // also waits for tail_id
  int id_base = 0;                           // id held in s_ids[0]
  auto lds_id = [&](int j) { return s_ids[min(j - id_base, kIdCap - 1)]; };
  Regs R[NBUF];
  int nid[NBUF];
  auto issue = [&](int j, int slot, int blk) {
    load_block(blk, j < nfull, kBlockTokens, R[slot]);
    if (j + NBUF - id_base >= kIdCap && j + NBUF < nfull) {
      fill_ids(j + NBUF);                    // rare: segments longer than kIdCap blocks
      id_base = j + NBUF;
    }
    nid[slot] = lds_id(j + NBUF);
  };
  Regs T;
  if constexpr (!PREFIX) load_block(__builtin_amdgcn_readfirstlane(tail_id), tail > 0, tail, T);
  __builtin_amdgcn_sched_barrier(0);
  // The prologue's loads stay in block order after the partial block's, so
  // each block's wait counts only the blocks issued after it.
#pragma unroll
  for (int s = 0; s + 1 < NBUF; ++s) {
    issue(s, s, __builtin_amdgcn_readfirstlane(lds_id(s)));
    __builtin_amdgcn_sched_barrier(0);
  }
  nid[NBUF - 1] = lds_id(NBUF - 1);
  if (tail > 0) process_block(std::integral_constant<bool, true>(), T, tail);
  for (int k = 0; k < nfull; k += NBUF) {
#pragma unroll
    for (int s = 0; s < NBUF; ++s) {
      constexpr int kLast = NBUF - 1;
      const int slot = (s + kLast) % NBUF;
      issue(k + s + kLast, slot, __builtin_amdgcn_readfirstlane(nid[slot]));
      __builtin_amdgcn_sched_barrier(0);
      if (s == 0 || k + s < nfull) process_block(full, R[s], kBlockTokens);
    }
  }
  finalize();
  } while (!PREFIX && next_segment(p, sg));
}

}  // namespace mfma
}  // namespace pa
