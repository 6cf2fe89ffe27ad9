// C ABI of libpa.so: argument validation, partition sizing, workspace
// layout and kernel dispatch.  Every check happens on the host before any
// launch; the library allocates nothing and keeps no state.
#include "pa.h"
#include "pa_internal.h"

#include <limits.h>

#include <mutex>

namespace {

using pa::kBlockTokens;

// Finest split of both decode kernels (tokens).  The waves stream balanced
// chunks of blocks sized on the device from the actual lengths
// (work_split.h), at least one partition long.
constexpr int kRunPartition = 256;
// Waves a decode launch aims at (256 CUs x 8 waves).
#ifndef PA_TARGET_WAVES
#define PA_TARGET_WAVES 2048
#endif
// (sequence, kv head) pairs from which the library gives each pair one wave
// over its whole context (no split, no merge).
#ifndef PA_DIRECT_PAIRS
#define PA_DIRECT_PAIRS 2048
#endif
constexpr int kMaxPartition = 1 << 18;      // largest partition accepted (tokens)
constexpr float kLog2e = 1.4426950408889634f;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

// Shape checks shared by every decode entry point.  0 = ok.
int check_decode_shapes(int max_blocks, int max_context_len, int batch, int q_heads,
                        int kv_heads, int head_dim, int block_size, int num_blocks,
                        int partition_size) {
  if (batch < 0 || q_heads <= 0 || kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0 ||
      max_blocks <= 0 || max_context_len < 0)
    return PA_ERR_SHAPE;
  if (batch > 65535 || kv_heads > 65535) return PA_ERR_SHAPE;   // grid y / z limits
  if (q_heads % kv_heads != 0) return PA_ERR_SHAPE;
  if (block_size != kBlockTokens) return PA_ERR_UNSUPPORTED;
  if ((long long)max_context_len > (long long)max_blocks * block_size) return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!supported_group(q_heads / kv_heads)) return PA_ERR_UNSUPPORTED;
  if (partition_size < 0 || partition_size % kBlockTokens != 0 || partition_size > kMaxPartition)
    return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// Library's partition size: the caller's if given.  Otherwise, when the
// (sequence, kv head) pairs alone reach the wave target, one
// partition covering the longest context (no split, no merge); else
// kRunPartition, with balanced chunks sized on the device.
int resolve_partition(int batch, int kv_heads, int max_context_len, int partition_size) {
  if (partition_size > 0) return partition_size;
  if ((long long)batch * kv_heads >= PA_DIRECT_PAIRS) {
    const int whole = (max(max_context_len, 1) + kBlockTokens - 1) / kBlockTokens * kBlockTokens;
    if (whole <= kMaxPartition) return max(whole, kRunPartition);
  }
  return kRunPartition;
}

int num_partitions(int max_context_len, int P) {
  const int n = (max_context_len + P - 1) / P;
  return n > 0 ? n : 1;
}

// Workspace: [header: int32 record mode, then per-sequence record counts
// from int kCountsAt on; 256-byte aligned][(m, l) records][fp16 o records], with
// n_part + 1 records per (sequence, query head) row: a balanced chunk may
// start inside a sequence's first partition, so a sequence can span one
// record more than it has partitions.
struct Records {
  size_t ml_offset, o_offset, total;
  int stride;   // records per row
};

Records record_layout(int batch, int q_heads, int head_dim, int n_part) {
  Records r;
  r.stride = n_part + 1;
  const size_t n = (size_t)batch * q_heads * r.stride;
  r.ml_offset = align_up((pa::kCountsAt + (size_t)batch) * sizeof(int), 256);
  r.o_offset = align_up(r.ml_offset + n * sizeof(float2), 256);
  r.total = r.o_offset + n * head_dim * sizeof(uint16_t);
  return r;
}

// Flattened block count of a batch must fit the kernels' int arithmetic.
bool blocks_fit(int batch, int max_context_len) {
  return (long long)batch * ((max_context_len + kBlockTokens - 1) / kBlockTokens) <= INT_MAX;
}

int status_of(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// Shared body of the decode entry points.  mode: 0 = full decode (direct
// when one partition, else partials + merge), 1 = partials only, 2 = check
// the arguments only (no workspace check, no launch).
int decode_common(int mode, void* out, float* lse_out, const void* q, const void* k_pool,
                  const void* v_pool, const float* k_scale, const float* v_scale, int kv,
                  const int32_t* block_table, int max_blocks, const int32_t* context_lens,
                  int max_context_len, int batch, int q_heads, int kv_heads, int head_dim,
                  int block_size, int num_blocks, float scale, int partition_size,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_pool || !v_pool || !block_table || !context_lens) return PA_ERR_NULL;
  if (mode != 1 && !out) return PA_ERR_NULL;
  if (kv != pa::kKvF16 && (!k_scale || !v_scale)) return PA_ERR_NULL;
  int st = check_decode_shapes(max_blocks, max_context_len, batch, q_heads, kv_heads, head_dim,
                               block_size, num_blocks, partition_size);
  if (st != PA_OK) return st;
  const int P = resolve_partition(batch, kv_heads, max_context_len, partition_size);
  const int n_part = num_partitions(max_context_len, P);
  if ((long long)n_part * batch * kv_heads > INT_MAX || !blocks_fit(batch, max_context_len))
    return PA_ERR_SHAPE;                     // 1-D grids, flattened block indices
  const bool direct = (mode == 0 && n_part == 1);
  const Records rec = record_layout(batch, q_heads, head_dim, n_part);
  if (mode == 2) return PA_OK;
  if (!direct) {
    if (!workspace) return PA_ERR_NULL;
    if (workspace_bytes < rec.total) return PA_ERR_WORKSPACE;
  }
  if (batch == 0) return PA_OK;

  pa::DecodeParams p = {};
  p.q = static_cast<const uint16_t*>(q);
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse_out;
  char* ws = static_cast<char*>(workspace);
  p.header = direct ? nullptr : reinterpret_cast<int*>(ws);
  p.part_ml = direct ? nullptr : reinterpret_cast<float2*>(ws + rec.ml_offset);
  p.part_o = direct ? nullptr : reinterpret_cast<uint16_t*>(ws + rec.o_offset);
  p.max_blocks = max_blocks;
  p.bt_stride = max_blocks;
  p.max_context_len = max_context_len;
  p.batch = batch;
  p.q_heads = q_heads;
  p.kv_heads = kv_heads;
  p.head_dim = head_dim;
  p.num_blocks = num_blocks;
  p.partition_size = P;
  p.n_part = n_part;
  p.rec_stride = rec.stride;
  p.scale_log2 = scale * kLog2e;
  p.direct = direct ? 1 : 0;
  p.target_waves = PA_TARGET_WAVES;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = status_of(pa::launch_decode(p, kv, s));
  if (st != PA_OK || direct || mode == 1) return st;

  pa::MergeParams mp = {};
  mp.header = p.header;
  mp.part_ml = p.part_ml;
  mp.part_o = p.part_o;
  mp.context_lens = context_lens;
  mp.out = p.out;
  mp.lse = lse_out;
  mp.batch = batch;
  mp.q_heads = q_heads;
  mp.head_dim = head_dim;
  mp.partition_size = P;
  mp.rec_stride = rec.stride;
  mp.max_context_len = max_context_len;
  return status_of(pa::launch_merge(mp, s));
}

// Shared-prefix workspace: [header][suffix (m, l) and o records, n_suf per
// row][prefix (m, l) records, n_pre per row][prefix o records].
struct PrefixRecords {
  Records suf;
  size_t pre_ml, pre_o, total;
};

PrefixRecords prefix_layout(int batch, int q_heads, int head_dim, int n_suf, int n_pre) {
  PrefixRecords r;
  r.suf = record_layout(batch, q_heads, head_dim, n_suf);
  const size_t n = (size_t)batch * q_heads * n_pre;
  r.pre_ml = align_up(r.suf.total, 256);
  r.pre_o = align_up(r.pre_ml + n * sizeof(float2), 256);
  r.total = r.pre_o + n * head_dim * sizeof(uint16_t);
  return r;
}

// Partition of the shared prefix: short enough that the prefix work has
// about PA_PREFIX_WAVES waves ((query tile, partition, kv head) items), at
// least one block, at most kRunPartition.  On 64 sequences sharing a
// 1024-token prefix at 32 kv heads (4 query tiles), with the suffix work in
// the same launch, the call took 56.1-56.3 us with 512 waves (256-token
// partitions), 59.4-59.9 us with 1024, 59.0-59.4 us with 256 (512-token
// partitions, the cap raised) and 83.7 us with 128; grouping the four tiles
// of a partition on one XCD changed nothing (alternating builds, one box).
#ifndef PA_PREFIX_WAVES
#define PA_PREFIX_WAVES 512
#endif
int prefix_partition(int batch, int q_heads, int kv_heads, int prefix_len) {
  const long long tiles = ((long long)batch * (q_heads / kv_heads) + 15) / 16;
  const long long per_part = tiles * kv_heads;   // waves per partition
  long long P = (long long)prefix_len * per_part / PA_PREFIX_WAVES;
  P = P / kBlockTokens * kBlockTokens;
  if (P < kBlockTokens) P = kBlockTokens;
  if (P > kRunPartition) P = kRunPartition;
  return (int)P;
}

// Partition of the private suffixes: the longest suffix split into at most
// PA_SUFFIX_SPLIT partitions, at least one block, at most kRunPartition.
// Suffixes are short and uneven (up to a few hundred tokens on top of a long
// shared prefix), so finer partitions even out the waves.  On 64 suffixes
// of 16..512 tokens at 32 kv heads, with the prefix work in the same launch,
// 128-token partitions (4) took the call to 67.8-68.1 us, against 68.9-69.2
// at 64 (8), 71.1-71.6 at 256 and 512, and 76.1-76.5 at 32 (16) (partition
// items; with the balanced chunks 4 and 8 measured alike, 2 slower).
#ifndef PA_SUFFIX_SPLIT
#define PA_SUFFIX_SPLIT 4
#endif
int suffix_partition(int suffix_max) {
  const int blocks = (suffix_max + kBlockTokens - 1) / kBlockTokens;
  const int P = (blocks + PA_SUFFIX_SPLIT - 1) / PA_SUFFIX_SPLIT * kBlockTokens;
  return P < kBlockTokens ? kBlockTokens : P > kRunPartition ? kRunPartition : P;
}

int check_prefix(int max_context_len, int prefix_len) {
  if (prefix_len <= 0 || prefix_len % kBlockTokens != 0 || prefix_len > max_context_len)
    return PA_ERR_SHAPE;
  return PA_OK;
}

// Decode over a prefix of prefix_len tokens shared by every sequence (table
// row 0's first prefix_len / 16 ids) plus each sequence's own suffix:
// partials over the suffixes, records over the prefix for all queries at
// once, then one merge of both.
int prefix_common(void* out, float* lse_out, const void* q, const void* k_pool,
                  const void* v_pool, const float* k_scale, const float* v_scale, int kv,
                  const int32_t* block_table, int max_blocks, const int32_t* context_lens,
                  int max_context_len, int batch, int q_heads, int kv_heads, int head_dim,
                  int block_size, int num_blocks, float scale, int prefix_len, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (!out || !q || !k_pool || !v_pool || !block_table || !context_lens) return PA_ERR_NULL;
  if (kv != pa::kKvF16 && (!k_scale || !v_scale)) return PA_ERR_NULL;
  int st = check_decode_shapes(max_blocks, max_context_len, batch, q_heads, kv_heads, head_dim,
                               block_size, num_blocks, 0);
  if (st != PA_OK) return st;
  if ((st = check_prefix(max_context_len, prefix_len)) != PA_OK) return st;
  const int suf_max = max_context_len - prefix_len;
  const int P = suffix_partition(suf_max);
  const int n_suf = num_partitions(suf_max, P);
  const int P_pre = prefix_partition(batch, q_heads, kv_heads, prefix_len);
  const int n_pre = num_partitions(prefix_len, P_pre);
  const long long queries = (long long)batch * (q_heads / kv_heads);
  const int tiles = (int)((queries + 15) / 16);
  if ((long long)n_suf * batch * kv_heads > INT_MAX ||
      (long long)tiles * n_pre * kv_heads > INT_MAX || !blocks_fit(batch, suf_max))
    return PA_ERR_SHAPE;
  const PrefixRecords rec = prefix_layout(batch, q_heads, head_dim, n_suf, n_pre);
  if (!workspace) return PA_ERR_NULL;
  if (workspace_bytes < rec.total) return PA_ERR_WORKSPACE;
  if (batch == 0) return PA_OK;

  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  pa::DecodeParams p = {};
  p.q = static_cast<const uint16_t*>(q);
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.batch = batch;
  p.q_heads = q_heads;
  p.kv_heads = kv_heads;
  p.head_dim = head_dim;
  p.num_blocks = num_blocks;
  p.partition_size = P;
  p.scale_log2 = scale * kLog2e;
  p.target_waves = PA_TARGET_WAVES;
  p.bt_stride = max_blocks;

  // Suffixes [prefix_len, L_b): records as pa_decode_partials would
  // write them for the shifted sequences.
  pa::DecodeParams ps = p;
  ps.header = reinterpret_cast<int*>(ws);
  ps.part_ml = reinterpret_cast<float2*>(ws + rec.suf.ml_offset);
  ps.part_o = reinterpret_cast<uint16_t*>(ws + rec.suf.o_offset);
  ps.token_offset = prefix_len;
  ps.max_blocks = max_blocks - prefix_len / kBlockTokens;
  ps.max_context_len = suf_max;
  ps.n_part = n_suf;
  ps.rec_stride = rec.suf.stride;
  // Balanced chunks over the suffixes even when the (sequence, kv head)
  // pairs alone reach the wave target: a wave target of one wave per
  // partition item caps the chunks at one partition, so the uneven suffixes
  // are cut into equal pieces instead of partitions that end early.  On 64
  // suffixes of 16..512 tokens at 32 kv heads the call took 66.1 against
  // 68.0 us with partition items (three alternating runs on one box).
  const long long suffix_items = (long long)n_suf * batch * kv_heads;
  if (suffix_items > ps.target_waves) ps.target_waves = (int)suffix_items;

  // Prefix: one record per (sequence, query head, prefix partition).
  pa::DecodeParams pp = p;
  pp.part_ml = reinterpret_cast<float2*>(ws + rec.pre_ml);
  pp.part_o = reinterpret_cast<uint16_t*>(ws + rec.pre_o);
  pp.max_blocks = prefix_len / kBlockTokens;
  pp.max_context_len = prefix_len;
  pp.partition_size = P_pre;
  pp.n_part = n_pre;
  pp.rec_stride = n_pre;
  pp.prefix_tiles = tiles;
  // Both record sets in one launch (decode_prefix.hip), then the merge.
  st = status_of(pa::launch_shared_prefix(ps, pp, kv, s));
  if (st != PA_OK) return st;

  pa::MergeParams mp = {};
  mp.header = ps.header;
  mp.part_ml = ps.part_ml;
  mp.part_o = ps.part_o;
  mp.context_lens = context_lens;
  mp.out = static_cast<uint16_t*>(out);
  mp.lse = lse_out;
  mp.batch = batch;
  mp.q_heads = q_heads;
  mp.head_dim = head_dim;
  mp.partition_size = P;
  mp.rec_stride = rec.suf.stride;
  mp.max_context_len = suf_max;
  mp.token_offset = prefix_len;
  mp.pre_ml = pp.part_ml;
  mp.pre_o = pp.part_o;
  mp.n_pre = n_pre;
  return status_of(pa::launch_merge(mp, s));
}

// Append workspace: the decode workspace, then one record per (sequence,
// query head) for the newest token: (m, l) float2 [B, Hq], fp16 u [B, Hq, D].
struct AppendRecords {
  Records part;
  size_t app_ml, app_o, total;
};

AppendRecords append_layout(int batch, int q_heads, int head_dim, int n_part) {
  AppendRecords r;
  r.part = record_layout(batch, q_heads, head_dim, n_part);
  const size_t n = (size_t)batch * q_heads;
  r.app_ml = align_up(r.part.total, 256);
  r.app_o = align_up(r.app_ml + n * sizeof(float2), 256);
  r.total = r.app_o + n * head_dim * sizeof(uint16_t);
  return r;
}

// Write each sequence's newest token (position context_lens[b] - 1) into its
// slot and decode over the whole context, in two launches: the partition
// kernel over tokens [0, L - 1) with the write and the new token's records
// in extra workgroups of the same grid, then the merge of both record sets.
int append_common(void* out, float* lse_out, const void* q, const void* k_new, const void* v_new,
                  void* k_pool, void* v_pool, float* k_scale, float* v_scale, int kv,
                  const int32_t* block_table, int max_blocks, const int32_t* context_lens,
                  int max_context_len, int batch, int q_heads, int kv_heads, int head_dim,
                  int block_size, int num_blocks, float scale, int partition_size,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!out || !q || !k_new || !v_new || !k_pool || !v_pool || !block_table || !context_lens)
    return PA_ERR_NULL;
  if (kv != pa::kKvF16 && (!k_scale || !v_scale)) return PA_ERR_NULL;
  int st = check_decode_shapes(max_blocks, max_context_len, batch, q_heads, kv_heads, head_dim,
                               block_size, num_blocks, partition_size);
  if (st != PA_OK) return st;
  const int P = resolve_partition(batch, kv_heads, max_context_len, partition_size);
  const int n_part = num_partitions(max_context_len, P);
  if ((long long)n_part * batch * kv_heads > INT_MAX || !blocks_fit(batch, max_context_len))
    return PA_ERR_SHAPE;
  const AppendRecords rec = append_layout(batch, q_heads, head_dim, n_part);
  if (!workspace) return PA_ERR_NULL;
  if (workspace_bytes < rec.total) return PA_ERR_WORKSPACE;
  if (batch == 0) return PA_OK;

  char* ws = static_cast<char*>(workspace);
  pa::DecodeParams p = {};
  p.q = static_cast<const uint16_t*>(q);
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.k_pool_w = k_pool;
  p.v_pool_w = v_pool;
  p.k_scale_w = k_scale;
  p.v_scale_w = v_scale;
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.header = reinterpret_cast<int*>(ws);
  p.part_ml = reinterpret_cast<float2*>(ws + rec.part.ml_offset);
  p.part_o = reinterpret_cast<uint16_t*>(ws + rec.part.o_offset);
  p.app_ml = reinterpret_cast<float2*>(ws + rec.app_ml);
  p.app_o = reinterpret_cast<uint16_t*>(ws + rec.app_o);
  p.max_blocks = max_blocks;
  p.bt_stride = max_blocks;
  p.max_context_len = max_context_len;
  p.len_trim = 1;
  p.batch = batch;
  p.q_heads = q_heads;
  p.kv_heads = kv_heads;
  p.head_dim = head_dim;
  p.num_blocks = num_blocks;
  p.partition_size = P;
  p.n_part = n_part;
  p.rec_stride = rec.part.stride;
  p.scale_log2 = scale * kLog2e;
  p.direct = 0;
  p.target_waves = PA_TARGET_WAVES;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = status_of(pa::launch_decode(p, kv, s));
  if (st != PA_OK) return st;

  pa::MergeParams mp = {};
  mp.header = p.header;
  mp.part_ml = p.part_ml;
  mp.part_o = p.part_o;
  mp.context_lens = context_lens;
  mp.out = static_cast<uint16_t*>(out);
  mp.lse = lse_out;
  mp.batch = batch;
  mp.q_heads = q_heads;
  mp.head_dim = head_dim;
  mp.partition_size = P;
  mp.rec_stride = rec.part.stride;
  mp.max_context_len = max_context_len;
  mp.len_trim = 1;
  mp.pre_ml = p.app_ml;
  mp.pre_o = p.app_o;
  mp.n_pre = 1;
  return status_of(pa::launch_merge(mp, s));
}

int check_write(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                const void* k_pool, const void* v_pool, int num_tokens, int num_blocks,
                int block_size, int kv_heads, int head_dim) {
  if (num_tokens < 0 || num_blocks <= 0 || kv_heads <= 0 || head_dim <= 0) return PA_ERR_SHAPE;
  if (num_tokens > 0 && (!k_new || !v_new || !slot_mapping)) return PA_ERR_NULL;
  if (!k_pool || !v_pool) return PA_ERR_NULL;
  if (block_size != kBlockTokens) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// Allocation-free decode (pa_decode_noalloc): the split-K records live in
// this file-scope device array instead of a caller workspace.  Each device
// the library runs on holds its own copy until the process ends.  In host
// code the name `scratch` is only a host-side stand-in for the symbol, never
// a device address: the device address comes from hipGetSymbolAddress, once
// per device, with that device current, and only that pointer is passed on.
constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];
void* g_scratch[kMaxDevices];
hipError_t g_scratch_status[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of the current device's copy of `scratch`.
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_status[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch[dev] = ptr;
  });
  if (g_scratch_status[dev] != hipSuccess || g_scratch[dev] == nullptr) return PA_ERR_HIP;
  *out = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK: success";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: inconsistent or non-positive shape";
    case PA_ERR_UNSUPPORTED:
      return "PA_ERR_UNSUPPORTED: block_size must be 16, head_dim 64/128, group 1/2/4/8/16, "
             "partition_size a multiple of 16";
    case PA_ERR_WORKSPACE:
      return "PA_ERR_WORKSPACE: workspace too small (pa_decode_noalloc: the records need more "
             "than its PA_NOALLOC_SCRATCH_BYTES of device scratch)";
    case PA_ERR_HIP: return "PA_ERR_HIP: kernel launch failed";
    default: return "unknown pa_status";
  }
}

int pa_write_kv(const void* k_new, const void* v_new, const int32_t* slot_mapping, void* k_pool,
                void* v_pool, int num_tokens, int num_blocks, int block_size, int kv_heads,
                int head_dim, void* stream) {
  int st = check_write(k_new, v_new, slot_mapping, k_pool, v_pool, num_tokens, num_blocks,
                       block_size, kv_heads, head_dim);
  if (st != PA_OK || num_tokens == 0) return st;
  pa::WriteParams p = {};
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.slots = slot_mapping;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.num_tokens = num_tokens;
  p.kv_heads = kv_heads;
  p.head_dim = head_dim;
  p.capacity = (long long)num_blocks * kBlockTokens;
  return status_of(pa::launch_write_kv(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

int write_q8(bool fp8, const void* k_new, const void* v_new, const int32_t* slot_mapping,
             void* k_pool, void* v_pool, float* k_scale, float* v_scale, int num_tokens,
             int num_blocks, int block_size, int kv_heads, int head_dim, void* stream) {
  int st = check_write(k_new, v_new, slot_mapping, k_pool, v_pool, num_tokens, num_blocks,
                       block_size, kv_heads, head_dim);
  if (st != PA_OK) return st;
  if (!k_scale || !v_scale) return PA_ERR_NULL;
  if (num_tokens == 0) return PA_OK;
  pa::WriteParams p = {};
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.slots = slot_mapping;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.num_tokens = num_tokens;
  p.kv_heads = kv_heads;
  p.head_dim = head_dim;
  p.capacity = (long long)num_blocks * kBlockTokens;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return status_of(fp8 ? pa::launch_write_kv_fp8(p, s) : pa::launch_write_kv_int8(p, s));
}

}  // namespace

extern "C" {

int pa_write_kv_int8(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                     int8_t* k_pool, int8_t* v_pool, float* k_scale, float* v_scale,
                     int num_tokens, int num_blocks, int block_size, int kv_heads, int head_dim,
                     void* stream) {
  return write_q8(false, k_new, v_new, slot_mapping, k_pool, v_pool, k_scale, v_scale,
                  num_tokens, num_blocks, block_size, kv_heads, head_dim, stream);
}

int pa_write_kv_fp8(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                    uint8_t* k_pool, uint8_t* v_pool, float* k_scale, float* v_scale,
                    int num_tokens, int num_blocks, int block_size, int kv_heads, int head_dim,
                    void* stream) {
  return write_q8(true, k_new, v_new, slot_mapping, k_pool, v_pool, k_scale, v_scale,
                  num_tokens, num_blocks, block_size, kv_heads, head_dim, stream);
}

int pa_copy_blocks(void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                   const int32_t* block_pairs, int num_pairs, int num_blocks, int block_size,
                   int kv_heads, int head_dim, int elem_bytes, void* stream) {
  if (!k_pool || !v_pool) return PA_ERR_NULL;
  if (num_pairs < 0 || num_blocks <= 0 || kv_heads <= 0 || head_dim <= 0) return PA_ERR_SHAPE;
  if (block_size != kBlockTokens) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (elem_bytes != 1 && elem_bytes != 2) return PA_ERR_UNSUPPORTED;
  if (elem_bytes == 1 && (!k_scale || !v_scale)) return PA_ERR_NULL;
  if (num_pairs > 0 && !block_pairs) return PA_ERR_NULL;
  if (num_pairs == 0) return PA_OK;
  pa::CopyParams p = {};
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.k_scale = elem_bytes == 1 ? k_scale : nullptr;
  p.v_scale = elem_bytes == 1 ? v_scale : nullptr;
  p.pairs = block_pairs;
  p.num_pairs = num_pairs;
  p.num_blocks = num_blocks;
  p.scales_per_block = kv_heads * kBlockTokens;
  p.block_bytes = (size_t)kBlockTokens * kv_heads * head_dim * elem_bytes;
  return status_of(pa::launch_copy_blocks(p, static_cast<hipStream_t>(stream)));
}

int pa_decode_partition_size(int batch, int q_heads, int kv_heads, int head_dim,
                             int max_context_len, int partition_size) {
  if (check_decode_shapes(1 << 30 >> 4, max_context_len, batch, q_heads, kv_heads, head_dim,
                          kBlockTokens, 1, partition_size) != PA_OK)
    return 0;
  return resolve_partition(batch, kv_heads, max_context_len, partition_size);
}

size_t pa_decode_workspace_size(int batch, int q_heads, int kv_heads, int head_dim,
                                int max_context_len, int partition_size) {
  const int P = pa_decode_partition_size(batch, q_heads, kv_heads, head_dim, max_context_len,
                                         partition_size);
  if (P == 0) return 0;
  return record_layout(batch, q_heads, head_dim, num_partitions(max_context_len, P)).total;
}

int pa_decode(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_table, int max_blocks, const int32_t* context_lens,
              int max_context_len, int batch, int q_heads, int kv_heads, int head_dim,
              int block_size, int num_blocks, float scale, int partition_size, void* workspace,
              size_t workspace_bytes, void* stream) {
  return decode_common(0, out, lse_out, q, k_pool, v_pool, nullptr, nullptr, pa::kKvF16, block_table,
                       max_blocks, context_lens, max_context_len, batch, q_heads, kv_heads,
                       head_dim, block_size, num_blocks, scale, partition_size, workspace,
                       workspace_bytes, stream);
}

int pa_decode_noalloc(void* out, float* lse_out, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_table, int max_blocks,
                      const int32_t* context_lens, int max_context_len, int batch, int q_heads,
                      int kv_heads, int head_dim, int block_size, int num_blocks, float scale,
                      int partition_size, void* stream) {
  // Argument checks and the size check come first: nothing touches the
  // device for a call that is refused.  0 bytes: direct mode.
  int st = decode_common(2, out, lse_out, q, k_pool, v_pool, nullptr, nullptr, pa::kKvF16,
                         block_table, max_blocks, context_lens, max_context_len, batch, q_heads,
                         kv_heads, head_dim, block_size, num_blocks, scale, partition_size,
                         nullptr, 0, stream);
  if (st != PA_OK || batch == 0) return st;
  // One partition covering every context: direct mode, no records.
  const int P = resolve_partition(batch, kv_heads, max_context_len, partition_size);
  const int n_part = num_partitions(max_context_len, P);
  const size_t need =
      n_part == 1 ? 0 : record_layout(batch, q_heads, head_dim, n_part).total;
  if (need > kScratchBytes) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_of_current_device(&ws);
    if (st != PA_OK) return st;
  }
  return decode_common(0, out, lse_out, q, k_pool, v_pool, nullptr, nullptr, pa::kKvF16,
                       block_table, max_blocks, context_lens, max_context_len, batch, q_heads,
                       kv_heads, head_dim, block_size, num_blocks, scale, partition_size, ws,
                       need, stream);
}

int pa_decode_int8(void* out, float* lse_out, const void* q, const int8_t* k_pool,
                   const int8_t* v_pool, const float* k_scale, const float* v_scale,
                   const int32_t* block_table, int max_blocks, const int32_t* context_lens,
                   int max_context_len, int batch, int q_heads, int kv_heads, int head_dim,
                   int block_size, int num_blocks, float scale, int partition_size,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(0, out, lse_out, q, k_pool, v_pool, k_scale, v_scale, pa::kKvI8, block_table,
                       max_blocks, context_lens, max_context_len, batch, q_heads, kv_heads,
                       head_dim, block_size, num_blocks, scale, partition_size, workspace,
                       workspace_bytes, stream);
}

int pa_decode_fp8(void* out, float* lse_out, const void* q, const uint8_t* k_pool,
                  const uint8_t* v_pool, const float* k_scale, const float* v_scale,
                  const int32_t* block_table, int max_blocks, const int32_t* context_lens,
                  int max_context_len, int batch, int q_heads, int kv_heads, int head_dim,
                  int block_size, int num_blocks, float scale, int partition_size,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(0, out, lse_out, q, k_pool, v_pool, k_scale, v_scale, pa::kKvF8,
                       block_table, max_blocks, context_lens, max_context_len, batch, q_heads,
                       kv_heads, head_dim, block_size, num_blocks, scale, partition_size,
                       workspace, workspace_bytes, stream);
}

size_t pa_decode_append_workspace_size(int batch, int q_heads, int kv_heads, int head_dim,
                                       int max_context_len, int partition_size) {
  const int P = pa_decode_partition_size(batch, q_heads, kv_heads, head_dim, max_context_len,
                                         partition_size);
  if (P == 0) return 0;
  return append_layout(batch, q_heads, head_dim, num_partitions(max_context_len, P)).total;
}

int pa_decode_append(void* out, float* lse_out, const void* q, const void* k_new,
                     const void* v_new, void* k_pool, void* v_pool, const int32_t* block_table,
                     int max_blocks, const int32_t* context_lens, int max_context_len, int batch,
                     int q_heads, int kv_heads, int head_dim, int block_size, int num_blocks,
                     float scale, int partition_size, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return append_common(out, lse_out, q, k_new, v_new, k_pool, v_pool, nullptr, nullptr,
                       pa::kKvF16, block_table, max_blocks, context_lens, max_context_len, batch,
                       q_heads, kv_heads, head_dim, block_size, num_blocks, scale, partition_size,
                       workspace, workspace_bytes, stream);
}

int pa_decode_append_int8(void* out, float* lse_out, const void* q, const void* k_new,
                          const void* v_new, int8_t* k_pool, int8_t* v_pool, float* k_scale,
                          float* v_scale, const int32_t* block_table, int max_blocks,
                          const int32_t* context_lens, int max_context_len, int batch,
                          int q_heads, int kv_heads, int head_dim, int block_size,
                          int num_blocks, float scale, int partition_size, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return append_common(out, lse_out, q, k_new, v_new, k_pool, v_pool, k_scale, v_scale,
                       pa::kKvI8, block_table, max_blocks, context_lens, max_context_len, batch,
                       q_heads, kv_heads, head_dim, block_size, num_blocks, scale, partition_size,
                       workspace, workspace_bytes, stream);
}

int pa_decode_append_fp8(void* out, float* lse_out, const void* q, const void* k_new,
                         const void* v_new, uint8_t* k_pool, uint8_t* v_pool, float* k_scale,
                         float* v_scale, const int32_t* block_table, int max_blocks,
                         const int32_t* context_lens, int max_context_len, int batch,
                         int q_heads, int kv_heads, int head_dim, int block_size,
                         int num_blocks, float scale, int partition_size, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return append_common(out, lse_out, q, k_new, v_new, k_pool, v_pool, k_scale, v_scale,
                       pa::kKvF8, block_table, max_blocks, context_lens, max_context_len, batch,
                       q_heads, kv_heads, head_dim, block_size, num_blocks, scale, partition_size,
                       workspace, workspace_bytes, stream);
}

int pa_decode_partials(const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_table, int max_blocks, const int32_t* context_lens,
                       int max_context_len, int batch, int q_heads, int kv_heads, int head_dim,
                       int block_size, int num_blocks, float scale, int partition_size,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(1, nullptr, nullptr, q, k_pool, v_pool, nullptr, nullptr, pa::kKvF16,
                       block_table, max_blocks, context_lens, max_context_len, batch, q_heads,
                       kv_heads, head_dim, block_size, num_blocks, scale, partition_size,
                       workspace, workspace_bytes, stream);
}

int pa_decode_partials_int8(const void* q, const int8_t* k_pool, const int8_t* v_pool,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_table, int max_blocks,
                            const int32_t* context_lens, int max_context_len, int batch,
                            int q_heads, int kv_heads, int head_dim, int block_size,
                            int num_blocks, float scale, int partition_size, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return decode_common(1, nullptr, nullptr, q, k_pool, v_pool, k_scale, v_scale, pa::kKvI8,
                       block_table, max_blocks, context_lens, max_context_len, batch, q_heads,
                       kv_heads, head_dim, block_size, num_blocks, scale, partition_size,
                       workspace, workspace_bytes, stream);
}

size_t pa_decode_shared_prefix_workspace_size(int batch, int q_heads, int kv_heads,
                                              int head_dim, int max_context_len,
                                              int prefix_len) {
  if (check_decode_shapes(1 << 30 >> 4, max_context_len, batch, q_heads, kv_heads, head_dim,
                          kBlockTokens, 1, 0) != PA_OK ||
      check_prefix(max_context_len, prefix_len) != PA_OK)
    return 0;
  return prefix_layout(batch, q_heads, head_dim,
                       num_partitions(max_context_len - prefix_len,
                                      suffix_partition(max_context_len - prefix_len)),
                       num_partitions(prefix_len,
                                      prefix_partition(batch, q_heads, kv_heads, prefix_len)))
      .total;
}

int pa_decode_shared_prefix(void* out, float* lse_out, const void* q, const void* k_pool,
                            const void* v_pool, const int32_t* block_table, int max_blocks,
                            const int32_t* context_lens, int max_context_len, int batch,
                            int q_heads, int kv_heads, int head_dim, int block_size,
                            int num_blocks, float scale, int prefix_len, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return prefix_common(out, lse_out, q, k_pool, v_pool, nullptr, nullptr, pa::kKvF16, block_table,
                       max_blocks, context_lens, max_context_len, batch, q_heads, kv_heads,
                       head_dim, block_size, num_blocks, scale, prefix_len, workspace,
                       workspace_bytes, stream);
}

int pa_decode_shared_prefix_int8(void* out, float* lse_out, const void* q, const int8_t* k_pool,
                                 const int8_t* v_pool, const float* k_scale,
                                 const float* v_scale, const int32_t* block_table,
                                 int max_blocks, const int32_t* context_lens,
                                 int max_context_len, int batch, int q_heads, int kv_heads,
                                 int head_dim, int block_size, int num_blocks, float scale,
                                 int prefix_len, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return prefix_common(out, lse_out, q, k_pool, v_pool, k_scale, v_scale, pa::kKvI8, block_table,
                       max_blocks, context_lens, max_context_len, batch, q_heads, kv_heads,
                       head_dim, block_size, num_blocks, scale, prefix_len, workspace,
                       workspace_bytes, stream);
}

int pa_decode_partials_fp8(const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_table, int max_blocks,
                           const int32_t* context_lens, int max_context_len, int batch,
                           int q_heads, int kv_heads, int head_dim, int block_size,
                           int num_blocks, float scale, int partition_size, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return decode_common(1, nullptr, nullptr, q, k_pool, v_pool, k_scale, v_scale, pa::kKvF8,
                       block_table, max_blocks, context_lens, max_context_len, batch, q_heads,
                       kv_heads, head_dim, block_size, num_blocks, scale, partition_size,
                       workspace, workspace_bytes, stream);
}

int pa_decode_shared_prefix_fp8(void* out, float* lse_out, const void* q, const uint8_t* k_pool,
                                const uint8_t* v_pool, const float* k_scale,
                                const float* v_scale, const int32_t* block_table,
                                int max_blocks, const int32_t* context_lens,
                                int max_context_len, int batch, int q_heads, int kv_heads,
                                int head_dim, int block_size, int num_blocks, float scale,
                                int prefix_len, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return prefix_common(out, lse_out, q, k_pool, v_pool, k_scale, v_scale, pa::kKvF8,
                       block_table, max_blocks, context_lens, max_context_len, batch, q_heads,
                       kv_heads, head_dim, block_size, num_blocks, scale, prefix_len, workspace,
                       workspace_bytes, stream);
}

int pa_merge_partials(void* out, float* lse_out, const int32_t* context_lens,
                      int max_context_len, int batch, int q_heads, int head_dim,
                      int partition_size, const void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!out || !context_lens || !workspace) return PA_ERR_NULL;
  if (batch < 0 || q_heads <= 0 || max_context_len < 0 || batch > 65535) return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (partition_size <= 0 || partition_size % kBlockTokens != 0 || partition_size > kMaxPartition)
    return PA_ERR_UNSUPPORTED;
  const int n_part = num_partitions(max_context_len, partition_size);
  const Records rec = record_layout(batch, q_heads, head_dim, n_part);
  if (workspace_bytes < rec.total) return PA_ERR_WORKSPACE;
  if (batch == 0) return PA_OK;
  pa::MergeParams mp = {};
  const char* ws = static_cast<const char*>(workspace);
  mp.header = reinterpret_cast<const int*>(ws);
  mp.part_ml = reinterpret_cast<const float2*>(ws + rec.ml_offset);
  mp.part_o = reinterpret_cast<const uint16_t*>(ws + rec.o_offset);
  mp.context_lens = context_lens;
  mp.out = static_cast<uint16_t*>(out);
  mp.lse = lse_out;
  mp.batch = batch;
  mp.q_heads = q_heads;
  mp.head_dim = head_dim;
  mp.partition_size = partition_size;
  mp.rec_stride = rec.stride;
  mp.max_context_len = max_context_len;
  return status_of(pa::launch_merge(mp, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
