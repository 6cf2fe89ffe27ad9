// Newest-token append inside a decode launch.
//
// A decode step writes each sequence's new token into its slot and then
// attends over the whole context, new token included (the zskr.cn ATB
// PagedAttention article, WriteKV in section "踩坑三", then the page-table
// attention of section "PagedAttention 的 Attention 计算修改"; the new
// token is position context_lens[b] - 1).  In append mode the partition
// work of the launch covers tokens [0, L - 1) only, so nothing in it reads
// the slot being written, and extra workgroups at the end of the same grid
// do the write and the new token's own record: one wave per (sequence, kv
// head) copies (fp16) or quantises (int8, FP8; quant.h) the K and V rows
// into the slot the block table gives for position L - 1, and for each of
// the G query heads stores the record (m = scale * log2(e) * q.k, l = 1,
// u = v) with k and v as the cache now holds them.  The merge kernel adds
// that record to the row's others.  The write's work thus overlaps the
// partition work instead of running as its own launch before it.
#pragma once

#include "pa_internal.h"
#include "quant.h"

namespace pa {

// One wave; lane holds head_dim elements lane * PER .. lane * PER + PER - 1.
// Sequences whose length is 0 or outside the contract get no record (the
// merge writes their rows); a table entry outside the pool skips the write
// and makes the record NaN.
template <int D, int G, int KV>
__device__ __forceinline__ void append_token(const DecodeParams& p, int pair) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int Hkv = p.kv_heads, Hq = p.q_heads;
  const int b = pair / Hkv, g = pair % Hkv;
  const int L = p.context_lens[b];
  if (L < 1 || L > p.max_context_len) return;
  const int t = L - 1;
  const int blk = p.block_table[(size_t)b * p.bt_stride + t / kBlockTokens];
  const bool bad = (unsigned)blk >= (unsigned)p.num_blocks;
  const size_t src = ((size_t)b * Hkv + g) * D + (size_t)lane * PER;
  const size_t dst = (((size_t)(bad ? 0 : blk) * kBlockTokens + t % kBlockTokens) * Hkv + g) * D +
                     (size_t)lane * PER;
  float kx[PER], vx[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    kx[e] = (float)__builtin_bit_cast(_Float16, p.k_new[src + e]);
    vx[e] = (float)__builtin_bit_cast(_Float16, p.v_new[src + e]);
  }
  if constexpr (KV == kKvF16) {
    if (!bad) {
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        static_cast<uint16_t*>(p.k_pool_w)[dst + e] = p.k_new[src + e];
        static_cast<uint16_t*>(p.v_pool_w)[dst + e] = p.v_new[src + e];
      }
    }
  } else {
    constexpr bool FP8 = KV == kKvF8;
    uint8_t kc[PER], vc[PER];
    const float ks = quantise_vals<PER, FP8>(kx, kc);
    const float vs = quantise_vals<PER, FP8>(vx, vc);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      kx[e] = code_value<FP8>(kc[e]) * ks;   // the values the cache now holds
      vx[e] = code_value<FP8>(vc[e]) * vs;
    }
    if (!bad) {
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        static_cast<uint8_t*>(p.k_pool_w)[dst + e] = kc[e];
        static_cast<uint8_t*>(p.v_pool_w)[dst + e] = vc[e];
      }
      if (lane == 0) {
        const size_t sidx = ((size_t)blk * Hkv + g) * kBlockTokens + t % kBlockTokens;
        p.k_scale_w[sidx] = ks;
        p.v_scale_w[sidx] = vs;
      }
    }
  }
  // The new token's record for each query head of the group.
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const size_t row = (size_t)b * Hq + g * G + i;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e)
      dot = fmaf((float)__builtin_bit_cast(_Float16, p.q[row * D + (size_t)lane * PER + e]), kx[e],
                 dot);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const _Float16 u = (_Float16)(bad ? nan : vx[e]);
      p.app_o[row * D + (size_t)lane * PER + e] = __builtin_bit_cast(uint16_t, u);
    }
    if (lane == 0) p.app_ml[row] = bad ? make_float2(nan, nan) : make_float2(dot * p.scale_log2, 1.0f);
  }
}

}  // namespace pa
