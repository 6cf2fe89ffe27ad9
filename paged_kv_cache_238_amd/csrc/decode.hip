// Paged-attention decode, split-K partition kernel (VALU form) for gfx950,
// used for query-head groups of 1 or 2 (larger groups use the matrix-core
// kernel in decode_mfma.hip).
//
// One workgroup = one (partition, kv head, sequence).  Its four wave64s walk
// the partition's 16-token blocks (wave w takes blocks w, w+4, ...), each
// keeping an online-softmax state for every query head of the kv head's
// group, then merge their states through LDS.  The result is either the
// final fp16 row (whole context in one partition) or one partition record
// (max, sum, unnormalised output) for the log-sum-exp merge kernel.
//
// Method: the zskr.cn article on ATB's PagedAttention, section
// "PagedAttention 的 Attention 计算修改" - per-page gather through the page
// table, dot of Q with each K row, running max with rescaling of the
// accumulator, V accumulation, final normalisation.  Differences from that
// listing: the running max is updated before the new term's exponent is
// taken, the max starts at -inf, a softmax scale is applied, accumulation is
// fp32, the output is indexed by head, and tail slots are masked.  The page
// table slice is staged in LDS once per workgroup (section "踩坑一").
// Query heads h = g*G .. g*G+G-1 share kv head g (discosf.com article
// "KV Cache 优化与显存管理", section "二、优化方向").
//
// Lane layout: a K/V row (one token, one kv head) of D elements is split
// over D/8 lanes holding 8 consecutive elements each (16 B for fp16, 8 B for
// int8), so one wave-wide load covers 64/(D/8) token rows.  Lanes holding
// the same token ("row group") reduce their partial dot products with DPP;
// every row group keeps its own running (max, sum, acc) so the hot loop has
// no cross-row traffic; row groups and waves are merged once at the end.
// Scores are kept in log2 units (scale * log2 e folded in), so exp is one
// v_exp_f32.
#include "pa_internal.h"

#include <type_traits>

namespace pa {
namespace {

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

__device__ __forceinline__ void buffer_load(uint4& dst, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  dst = make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void buffer_load(uint2& dst, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
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
__device__ __forceinline__ void to_f32(const uint2& c, float (&f)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = (float)(int)(int8_t)(c.x >> (8 * e));
#pragma unroll
  for (int e = 0; e < 4; ++e) f[4 + e] = (float)(int)(int8_t)(c.y >> (8 * e));
}

template <int D, int G, bool I8>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(const DecodeParams p) {
  constexpr int LPR = D / 8;                 // lanes per token row
  constexpr int RPW = 64 / LPR;              // token rows per wave load
  constexpr int NL = kBlockTokens / RPW;     // wave loads per block
  using Chunk = typename KvChunk<I8>::T;
  constexpr int ESZ = I8 ? 1 : 2;
  extern __shared__ float smem[];

  // 1-D grid, partition slowest (see the matrix-core kernel): consecutive
  // workgroups, which land on different XCDs, are different (sequence, kv
  // head) pairs of one partition index.
  const int pairs = p.batch * p.kv_heads;
  const int part = blockIdx.x / pairs;
  const int b = (blockIdx.x % pairs) / p.kv_heads, g = (blockIdx.x % pairs) % p.kv_heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int r = lane / LPR, c = lane % LPR;
  const int Hq = p.q_heads, Hkv = p.kv_heads;
  const int h0 = g * G;

  if (!p.direct && blockIdx.x == 0 && tid == 0) p.header[0] = 1;   // one partition per record
  const int L = p.context_lens[b];
  const int P = p.partition_size;
  const int t_begin = part * P;
  if (L < 0 || L > p.max_context_len) {
    // broken metadata: NaN rows, written once
    if (part == 0) {
      for (int i = tid; i < G * D; i += kThreads) {
        const int h = h0 + i / D, d = i % D;
        const size_t row = (size_t)b * Hq + h;
        if (p.direct) {
          p.out[row * D + d] = 0x7E00;
          if (d == 0 && p.lse) p.lse[row] = __builtin_nanf("");
        }
      }
    }
    return;
  }
  if (t_begin >= L) {
    if (p.direct && part == 0) {   // L == 0: zero row, lse = -inf
      for (int i = tid; i < G * D; i += kThreads) {
        const int h = h0 + i / D, d = i % D;
        const size_t row = (size_t)b * Hq + h;
        p.out[row * D + d] = 0;
        if (d == 0 && p.lse) p.lse[row] = kNegInf;
      }
    }
    return;
  }
  const int t_end = min(t_begin + P, L);
  const int ntok = t_end - t_begin;
  const int nblk = (ntok + kBlockTokens - 1) / kBlockTokens;
  const int j0 = t_begin / kBlockTokens;

  // Stage this partition's slice of the block table in LDS, once.
  int* s_ids = reinterpret_cast<int*>(smem);
  {
    const int32_t* row = p.block_table + (size_t)b * p.max_blocks + j0;
    for (int i = tid; i < nblk; i += kThreads) s_ids[i] = row[i];
  }
  __syncthreads();

  // Query slice of every head in the group: elements c*8 .. c*8+7.
  uint4 qraw[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
    qraw[hh] = *reinterpret_cast<const uint4*>(p.q + ((size_t)b * Hq + h0 + hh) * D + c * 8);
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

  struct Regs {
    Chunk k[NL];
    Chunk v[NL];
    float ks[NL];
    float vs[NL];
  };

  // Issue every K load of block jj, then every V load (V arrives while the
  // scores are computed).  real == false: a prefetch past the last block;
  // its loads are out of range of an empty resource and fetch nothing.
  const uint32_t scale_blk_bytes = (uint32_t)kBlockTokens * Hkv * sizeof(float);
  auto load_block = [&](int jj, bool real, Regs& R) {
    int blk = __builtin_amdgcn_readfirstlane(s_ids[real ? jj : 0]);
    if ((unsigned)blk >= (unsigned)p.num_blocks) {
      if (real) bad_blk = true;   // the result becomes NaN; read nothing
      real = false;
      blk = 0;
    }
    const uint32_t nbytes = real ? blk_bytes : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (size_t)blk * blk_bytes, nbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (size_t)blk * blk_bytes, nbytes);
#pragma unroll
    for (int i = 0; i < NL; ++i) buffer_load(R.k[i], rk, lane_off[i]);
#pragma unroll
    for (int i = 0; i < NL; ++i) buffer_load(R.v[i], rv, lane_off[i]);
    if constexpr (I8) {
      const uint32_t sbytes = real ? scale_blk_bytes : 0u;
      const __amdgpu_buffer_rsrc_t rks = make_rsrc(p.k_scale + (size_t)blk * kBlockTokens * Hkv, sbytes);
      const __amdgpu_buffer_rsrc_t rvs = make_rsrc(p.v_scale + (size_t)blk * kBlockTokens * Hkv, sbytes);
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
      if constexpr (I8) to_f32(R.k[i], kf);
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
    float vf[NL][8];
    float vsc[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      to_f32(R.v[i], vf[i]);
      vsc[i] = R.vs[i];
      if constexpr (TAIL) {
        if (r + RPW * i >= valid) {   // masked row: value and its scale may be NaN
#pragma unroll
          for (int e = 0; e < 8; ++e) vf[i][e] = 0.f;
          vsc[i] = 0.f;
        }
      }
    }
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
        const float pr = fast_exp2(s[hh][i] - m_use);
        l[hh] += pr;
        const float pv = I8 ? pr * vsc[i] : pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(pv, vf[i][e], acc[hh][e]);
      }
      m[hh] = m_new;
    }
  };

  // Full blocks of this wave: w, w+4, ...  Two register sets alternate so
  // the loads of the next block are in flight while the current one is
  // reduced.  Loads sit outside every branch (prefetches past the end read
  // nothing) and all branches are wave-uniform, so the waits stay exact.
  const int nfull = ntok / kBlockTokens;
  const int nmine = nfull > w ? (nfull - w + kWaves - 1) / kWaves : 0;
  if (nmine > 0) {
    std::integral_constant<bool, false> full;
    Regs A, B;
    load_block(w, true, A);
    for (int k = 0; k < nmine; k += 2) {
      load_block(w + (k + 1) * kWaves, k + 1 < nmine, B);
      __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the math
      process_block(full, A, kBlockTokens);
      load_block(w + (k + 2) * kWaves, k + 2 < nmine, A);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 1 < nmine) process_block(full, B, kBlockTokens);
    }
  }
  // The partial last block (only in a sequence's last partition).
  const int tail = ntok - nfull * kBlockTokens;
  if (tail > 0 && w == nfull % kWaves) {
    Regs T;
    load_block(nfull, true, T);
    process_block(std::integral_constant<bool, true>(), T, tail);
  }

  // Merge the RPW row groups of this wave.
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float M = m[hh];
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float f = fast_exp2(m[hh] - ((M == kNegInf) ? 0.f : M));
    float lw = l[hh] * f;
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) lw += __shfl_xor(lw, off);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float o = acc[hh][e] * f;
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) o += __shfl_xor(o, off);
      acc[hh][e] = o;
    }
    m[hh] = M;
    l[hh] = lw;
  }

  // Merge the waves through LDS (reusing the block-id area).
  __syncthreads();
  float* s_m = smem;                          // [kWaves][G]
  float* s_l = s_m + kWaves * G;              // [kWaves][G]
  float* s_o = s_l + kWaves * G;              // [kWaves][G][D]
  int* s_bad = reinterpret_cast<int*>(s_o + kWaves * G * D);   // [kWaves]
  if (r == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[(w * G + hh) * D + c * 8 + e] = acc[hh][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      s_m[w * G + hh] = m[hh];
      s_l[w * G + hh] = l[hh];
    }
    s_bad[w] = bad_blk ? 1 : 0;
  }
  __syncthreads();
  const bool any_bad = s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3];
  for (int i = tid; i < G * D; i += kThreads) {
    const int hh = i / D, d = i % D;
    float M = s_m[hh];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww * G + hh]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = fast_exp2(s_m[ww * G + hh] - Mu);
      den = fmaf(s_l[ww * G + hh], f, den);
      num = fmaf(s_o[(ww * G + hh) * D + d], f, num);
    }
    if (any_bad) {
      num = den = M = __builtin_nanf("");
    }
    const size_t row = (size_t)b * Hq + h0 + hh;
    if (p.direct) {
      p.out[row * D + d] = f32_to_f16_bits(num / den);
      if (d == 0 && p.lse) p.lse[row] = (M + __log2f(den)) * kLn2;
    } else {
      const size_t rec = row * p.n_part + part;
      p.part_o[rec * D + d] = num;
      if (d == 0) p.part_ml[rec] = make_float2(M, den);
    }
  }
}

template <int D, int G, bool I8>
hipError_t launch_one(const DecodeParams& p, hipStream_t stream) {
  const int max_ids = p.partition_size / kBlockTokens;
  const size_t lds_ids = (size_t)max_ids * sizeof(int);
  const size_t lds_merge = (size_t)kWaves * G * (D + 2) * sizeof(float) + kWaves * sizeof(int);
  const size_t lds = lds_ids > lds_merge ? lds_ids : lds_merge;
  const unsigned grid = (unsigned)p.n_part * p.batch * p.kv_heads;
  hipLaunchKernelGGL((decode_valu_kernel<D, G, I8>), dim3(grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

template <int D, bool I8>
hipError_t dispatch_group(const DecodeParams& p, hipStream_t stream) {
  switch (p.q_heads / p.kv_heads) {
    case 1: return launch_one<D, 1, I8>(p, stream);
    case 2: return launch_one<D, 2, I8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_valu(const DecodeParams& p, bool int8, hipStream_t stream) {
  if (p.head_dim == 128) return int8 ? dispatch_group<128, true>(p, stream) : dispatch_group<128, false>(p, stream);
  if (p.head_dim == 64) return int8 ? dispatch_group<64, true>(p, stream) : dispatch_group<64, false>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, bool int8, hipStream_t stream) {
  const int group = p.q_heads / p.kv_heads;
  if (group >= 4) return launch_decode_mfma(p, int8, stream);
  return launch_decode_valu(p, int8, stream);
}

}  // namespace pa
