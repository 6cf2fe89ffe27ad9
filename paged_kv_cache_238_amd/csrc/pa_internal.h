// Internal interface between the C-ABI layer (pa_api.hip) and the kernel
// launchers.  Not installed; no torch types anywhere.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockTokens = 16;   // tokens per physical KV block

// Workspace header (int32): [0] = record mode (1: record r of a row covers
// partition r; 0: balanced chunks, per-sequence record counts from
// header[kCountsAt + b]).  The header takes 256 bytes plus the counts,
// rounded up to 256 bytes.
constexpr int kCountsAt = 64;

// KV cache element formats.  The 8-bit ones carry fp32 scales per (token,
// kv head), laid out [num_blocks, kv_heads, 16].
enum : int {
  kKvF16 = 0,   // fp16 values
  kKvI8 = 1,    // int8 codes
  kKvF8 = 2,    // OCP FP8 E4M3 codes
};

// Everything one decode launch needs.  Pointers are device pointers.
struct DecodeParams {
  const uint16_t* q;          // fp16 [B, Hq, D]
  const void* k_pool;         // fp16, int8 or fp8 [NB, 16, Hkv, D]
  const void* v_pool;
  const float* k_scale;       // 8-bit pools only: fp32 [NB, Hkv, 16]
  const float* v_scale;
  const int32_t* block_table; // [B, max_blocks]
  const int32_t* context_lens;// [B]
  uint16_t* out;              // fp16 [B, Hq, D]  (direct mode)
  float* lse;                 // fp32 [B, Hq] or null (direct mode)
  float2* part_ml;            // [rec_stride, B, Hq] (split mode; record-major)
  uint16_t* part_o;           // fp16 [rec_stride, B, Hq, D], normalised (split mode)
  int max_blocks;             // table entries per row from token_offset on
  int bt_stride;              // table row stride (entries)
  int token_offset;           // tokens [0, token_offset) of every sequence are
                              // skipped (multiple of 16): lengths and table rows
                              // are read past them
  int max_context_len;        // bound on context_lens - token_offset
  int len_trim;               // tokens dropped from the end of every sequence
                              // (1 when the launch appends the newest token itself)
  int batch, q_heads, kv_heads, head_dim, num_blocks;
  int partition_size;         // tokens, multiple of 16
  int n_part;                 // ceil(max_context_len / partition_size)
  int rec_stride;             // records per (sequence, query head) row: n_part + 1
  float scale_log2;           // scale * log2(e)
  int direct;                 // 1: n_part == 1, write out/lse directly
  int target_waves;           // waves a launch aims at (locate_work, work_split.h)
  int* header;                // split mode: workspace header (kCountsAt)
  // Append mode: workgroups from main_groups on write each sequence's new
  // token (position context_lens[b] - 1) from k_new / v_new into its slot and
  // emit that token's record into app_ml / app_o ([B, Hq], one record per row).
  int main_groups;            // workgroups of the partition work (append mode)
  const uint16_t* k_new;      // fp16 [B, Hkv, D]
  const uint16_t* v_new;
  void* k_pool_w;             // the pools and (8-bit) scales the append writes
  void* v_pool_w;
  float* k_scale_w;
  float* v_scale_w;
  float2* app_ml;
  uint16_t* app_o;
  // Shared-prefix mode (matrix-core kernel): the stream is table row 0 over
  // max_context_len tokens (the prefix), one partition per run, and the 16
  // query slots of a wave are queries of different sequences: query
  // qi = tile * 16 + slot is head g * G + qi % G of sequence qi / G.
  int prefix_tiles;           // ceil(batch * G / 16)
  int prefix_tile_waves;      // 1: the waves of a prefix workgroup are consecutive
                              // query tiles of one kv head (they stream the same
                              // K/V lines together); 0: kv heads of one tile
};

struct MergeParams {
  const int* header;          // record mode and per-sequence counts (kCountsAt)
  const float2* part_ml;
  const uint16_t* part_o;     // fp16 normalised outputs
  const int32_t* context_lens;
  uint16_t* out;
  float* lse;
  int batch, q_heads, head_dim;
  int partition_size, rec_stride, max_context_len;
  int token_offset;           // records cover tokens [token_offset, L - len_trim)
  int len_trim;               // 1: the row's last token is in the second record set
  // Optional second record set (shared prefix): n_pre records per row, all
  // present.  Null when absent.
  const float2* pre_ml;
  const uint16_t* pre_o;
  int n_pre;
};

struct WriteParams {
  const uint16_t* k_new;      // fp16 [T, Hkv, D]
  const uint16_t* v_new;
  const int32_t* slots;       // [T]
  void* k_pool;
  void* v_pool;
  float* k_scale;             // 8-bit pools only
  float* v_scale;
  int num_tokens, kv_heads, head_dim;
  long long capacity;         // num_blocks * 16 slots
};

struct CopyParams {
  void* k_pool;               // any element type; blocks are byte runs
  void* v_pool;
  float* k_scale;             // 8-bit pools: [NB, Hkv, 16]; null for fp16
  float* v_scale;
  const int32_t* pairs;       // [num_pairs][2]: (src block, dst block)
  int num_pairs, num_blocks;
  int scales_per_block;       // kv_heads * 16
  size_t block_bytes;         // 16 * kv_heads * head_dim * element bytes
};

// Length of sequence b as the partition work sees it.
__device__ __forceinline__ int seq_len(const DecodeParams& p, int b) {
  return p.context_lens[b] - p.token_offset - p.len_trim;
}

// Workgroups of a decode launch with `wpg` kv heads per workgroup: one per
// sequence in direct mode; n_part * batch partition items when batch *
// kv_heads reaches the wave target; otherwise at most target_waves /
// kv_heads balanced chunks (locate_work in work_split.h), and no more than
// the partitions could fill, each times the head groups.
inline unsigned decode_workgroups(const DecodeParams& p, int wpg) {
  const long long groups = p.kv_heads / wpg;
  if (p.direct) return (unsigned)(p.batch * groups);
  const long long full = (long long)p.n_part * p.batch;
  if ((long long)p.batch * p.kv_heads >= p.target_waves) return (unsigned)(full * groups);
  long long chunks = p.target_waves / p.kv_heads;
  if (chunks < 1) chunks = 1;
  return (unsigned)((full < chunks ? full : chunks) * groups);
}

// Extra workgroups of an append-mode launch: one wave per (sequence, kv head).
inline unsigned append_workgroups(const DecodeParams& p, int wpg) {
  if (p.k_new == nullptr) return 0;
  return (unsigned)(((long long)p.batch * p.kv_heads + wpg - 1) / wpg);
}

// Launchers return hipSuccess or the launch error.  `kv` is the cache
// format (kKvF16, kKvI8, kKvF8).
// Group size 1 or 2: VALU kernel; 4, 8 or 16: matrix-core kernel.
hipError_t launch_decode(const DecodeParams& p, int kv, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeParams& p, int kv, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeParams& p, int kv, hipStream_t stream);
// Suffix partition work and prefix work of the shared-prefix call in one launch.
hipError_t launch_shared_prefix(const DecodeParams& ps, const DecodeParams& pp, int kv,
                                hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);
hipError_t launch_write_kv(const WriteParams& p, hipStream_t stream);
hipError_t launch_write_kv_int8(const WriteParams& p, hipStream_t stream);
hipError_t launch_write_kv_fp8(const WriteParams& p, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t stream);

}  // namespace pa
