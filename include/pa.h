/*
 * pa.h - paged-attention decode over a block-paged KV cache, for AMD MI355X
 * (gfx950).  C ABI of libpa.so.
 *
 * Sources (the three web pages on KV-cache paging):
 *   [ATB-KV]  adg.csdn.net article on ATB's KV Cache management: section
 *             "Paged KV Cache" (fixed 16-token blocks allocated on demand),
 *             "Prefix Caching" (one prompt prefix's blocks shared by many
 *             requests), "显存碎片问题" (scattered blocks).
 *   [KV-OPT]  discosf.com article "KV Cache 优化与显存管理": section
 *             "二、优化方向" (logically contiguous tokens on physically
 *             non-contiguous pages; grouped query heads sharing one K/V
 *             head; FP16 -> INT8 cache), section "三、实现示例"
 *             (PhysicalPagePool.write_page, KVCacheQuantizer per_channel
 *             quantize / dequantize).
 *   [ATB-PA]  zskr.cn article on ATB's PagedAttention: section
 *             "PagedAttention 的 Attention 计算修改" (PagedAttentionKernel:
 *             Q [batch, num_heads, d_head], K/V pages, page_table
 *             [request, max_pages], output [batch, num_heads, d_head];
 *             per-page online softmax), "踩坑一" (page table staged on chip
 *             once), "踩坑三" (WriteKV appends a token's K, V into its page).
 *
 * Layout (all tensors C-contiguous, every pointer a device pointer owned by
 * the caller unless stated otherwise):
 *   q, out        fp16  [batch, q_heads, head_dim]
 *   k_pool,v_pool fp16 or int8 [num_blocks, block_size, kv_heads, head_dim]
 *   k_scale,      fp32  [num_blocks, kv_heads, block_size]   (int8 pools:
 *   v_scale             one scale per token and kv head; the 16 scales of
 *                       one (block, kv head) are adjacent, one 64-byte line)
 *   block_table   int32 [batch, max_blocks]; entry j of row b is the physical
 *                       block holding logical tokens 16j .. 16j+15 of b
 *   context_lens  int32 [batch]; tokens of sequence b, including the newest
 *   slot_mapping  int32 [num_tokens]; slot = block * block_size + offset
 *   lse_out       fp32  [batch, q_heads] natural-log log-sum-exp of the
 *                       scaled scores (optional, may be NULL)
 * Query head h reads kv head h / (q_heads / kv_heads).
 *
 * Behaviour common to every entry point:
 *   - block_size must be 16, head_dim 64 or 128, q_heads / kv_heads in
 *     {1, 2, 4, 8, 16}.
 *   - Argument errors return a nonzero pa_status before anything is
 *     launched.  Launch failures return PA_ERR_HIP.  Device-side faults
 *     surface at the caller's next synchronisation, as in HIP.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = null stream) and
 *     is asynchronous.  The library allocates no memory, keeps no state
 *     between calls and retains no pointer after it returns (the one
 *     exception: pa_decode_noalloc's per-device scratch array, below).
 *     Nothing throws or aborts across this ABI.
 *   - Caller contracts that are not checked on the host (they would need a
 *     device synchronisation): 0 <= block_table[b][j] < num_blocks for
 *     j < ceil(L_b / 16); 0 <= L_b <= max_context_len.  The kernels check
 *     both on the device without faulting: a sequence that breaks either
 *     gets NaN in every element of its output rows.  Entries past
 *     ceil(L_b / 16) are never read.  Tokens t >= L_b of the last block
 *     never influence the output, whatever those slots hold.
 *   - Results are deterministic: no floating-point atomics, fixed
 *     reduction order for a given (shape, partition_size).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* non-positive size, q_heads % kv_heads != 0,
                             max_context_len > max_blocks * block_size, ... */
  PA_ERR_UNSUPPORTED = 3, /* block_size != 16, head_dim not 64/128, group not
                             in {1,2,4,8,16}, partition_size not a positive
                             multiple of 16 (or 0) */
  PA_ERR_WORKSPACE = 4,   /* workspace smaller than pa_decode_workspace_size
                             (the library never allocates) */
  PA_ERR_HIP = 5          /* a kernel launch failed */
} pa_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* pa_status_string(int status);

/*
 * KV write ("reshape and cache"): for every i < num_tokens with
 * slot_mapping[i] >= 0, copy the rows k_new[i] / v_new[i] ([kv_heads,
 * head_dim] fp16) into k_pool / v_pool at block slot_mapping[i] / 16,
 * offset slot_mapping[i] % 16.  [KV-OPT] "三、实现示例" write_page;
 * [ATB-PA] "踩坑三" WriteKV.
 *   k_new, v_new  fp16 [num_tokens, kv_heads, head_dim]
 *   k_pool, v_pool fp16 [num_blocks, block_size, kv_heads, head_dim]
 * A byte copy: the written rows equal the inputs bit for bit and no other
 * byte of either pool changes.  Negative slots are skipped; slots >=
 * num_blocks * 16 are skipped too (never written).  Slots must be unique
 * and lie in blocks no other sequence shares (copy-on-write is the
 * caller's job, [ATB-PA] "踩坑三"); duplicates race.  num_tokens == 0 is a
 * no-op.  Ordered before a following pa_decode on the same stream.
 */
int pa_write_kv(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                void* k_pool, void* v_pool, int num_tokens, int num_blocks,
                int block_size, int kv_heads, int head_dim, void* stream);

/*
 * KV write into an int8 pool: each new row [head_dim] of k_new / v_new is
 * quantised with its own scale, absmax(|x|) / 127 in fp32 (a zero scale
 * becomes 1.0), codes = clip(round-half-even(x / scale), -128, 127), and
 * codes and scale are stored at the slot.  [KV-OPT] "三、实现示例"
 * KVCacheQuantizer.quantize, per_channel branch (last axis = head_dim);
 * "二、优化方向" FP16 -> INT8 cache.  Same slot rules as pa_write_kv.
 *   k_pool, v_pool int8 [num_blocks, block_size, kv_heads, head_dim]
 *   k_scale, v_scale fp32 [num_blocks, kv_heads, block_size]
 */
int pa_write_kv_int8(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                     int8_t* k_pool, int8_t* v_pool, float* k_scale, float* v_scale,
                     int num_tokens, int num_blocks, int block_size, int kv_heads,
                     int head_dim, void* stream);

/*
 * FP8 KV cache.  The discosf.com article "KV Cache 优化与显存管理" (section
 * "二、优化方向") names FP8 beside INT8 as a KV-cache precision that halves
 * its memory, without a format or a scale rule.  This library's FP8 is the
 * OCP FP8 E4M3 format (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; largest finite value 448; S.1111.111 is NaN), which gfx950 converts
 * natively.  Pools hold raw codes, uint8 [num_blocks, block_size, kv_heads,
 * head_dim]; scales are fp32 [num_blocks, kv_heads, block_size] as for int8,
 * and an element's value is E4M3(code) * scale.
 *
 * pa_write_kv_fp8: the quantising write, per (token, kv head) row, by the
 * per_channel rule of the int8 write with 448 in place of 127: scale =
 * absmax / 448 in fp32 (IEEE division; zero -> 1.0), code = the E4M3 value
 * nearest to x / scale (fp32 IEEE division), ties to the even code,
 * magnitudes at or above 448 saturating to 448.  Arguments, skip rules and
 * status codes as for pa_write_kv_int8.
 */
int pa_write_kv_fp8(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                    uint8_t* k_pool, uint8_t* v_pool, float* k_scale, float* v_scale,
                    int num_tokens, int num_blocks, int block_size, int kv_heads,
                    int head_dim, void* stream);

/*
 * Block copy for copy-on-write.  The zskr.cn article on ATB's PagedAttention
 * (section "踩坑三") updates a page that several requests share by taking a
 * fresh page, copying the old page into it and only then writing the new
 * token; the caller's block manager decides which blocks to copy
 * (reference counts, section "踩坑二"), this call copies them on the device.
 *
 *   k_pool, v_pool   the pools, [num_blocks, block_size, kv_heads, head_dim]
 *                    of elem_bytes each (2: fp16; 1: int8 or fp8 codes)
 *   k_scale, v_scale fp32 [num_blocks, kv_heads, block_size]; required when
 *                    elem_bytes is 1 (copied with their blocks), ignored
 *                    when it is 2
 *   block_pairs      int32 [num_pairs][2] on the device: (src, dst) block
 *                    ids; every element of block src (K, V and scales) is
 *                    copied to block dst.  A pair naming a block outside
 *                    [0, num_blocks) is skipped.  Caller contract: the dst
 *                    blocks are distinct and none is also a src of the same
 *                    call (the copies run concurrently).
 * Returns PA_OK, PA_ERR_NULL, PA_ERR_SHAPE (negative counts, non-positive
 * sizes) or PA_ERR_UNSUPPORTED (block_size != 16, head_dim not 64/128,
 * elem_bytes not 1/2); num_pairs = 0 is a no-op.  Asynchronous on `stream`.
 */
int pa_copy_blocks(void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                   const int32_t* block_pairs, int num_pairs, int num_blocks, int block_size,
                   int kv_heads, int head_dim, int elem_bytes, void* stream);

/*
 * Partition size the library uses for these shapes when partition_size is
 * 0, else partition_size itself (a multiple of 16).  The library's choice:
 * 256 tokens, the finest split, with the work cut into balanced chunks on
 * the device (see the workspace layout below); or, when batch * kv_heads
 * alone reaches 2048 (enough waves to fill the GPU), one partition covering
 * max_context_len rounded up to 16, so no merge runs.  Returns 0 on invalid
 * arguments.
 */
int pa_decode_partition_size(int batch, int q_heads, int kv_heads, int head_dim,
                             int max_context_len, int partition_size);

/*
 * Bytes of device workspace pa_decode / pa_decode_int8 / pa_decode_fp8 and
 * pa_decode_partials* need for these shapes: the layout of the partial
 * records (below) for ceil(max_context_len / P) partitions, P the resolved
 * partition size.  When that is one partition, pa_decode* run in direct
 * mode and read no workspace (NULL is accepted); pa_decode_partials* still
 * write records.  Returns 0 on invalid arguments.
 */
size_t pa_decode_workspace_size(int batch, int q_heads, int kv_heads, int head_dim,
                                int max_context_len, int partition_size);

/*
 * Decode attention, one query token per sequence:
 *   out[b,h,:] = sum_{t<L_b} softmax_t(scale * q[b,h,:] . K_b[t]) V_b[t]
 * with K_b[t] = k_pool[block_table[b][t/16], t%16, h/G, :] (V likewise).
 * [ATB-PA] "PagedAttention 的 Attention 计算修改" (per-page gather and
 * online softmax; here with the scale, the head index and an fp32
 * accumulator); [KV-OPT] "二、优化方向" (GQA grouping).
 *   max_context_len  host-side upper bound on context_lens (sizes the grid;
 *                    no device-to-host read); <= max_blocks * 16
 *   scale            usually 1/sqrt(head_dim)
 *   partition_size   granularity of the split-K work in tokens, a multiple
 *                    of 16; 0 = library's choice (pa_decode_partition_size).
 *                    With the balanced split (batch * kv_heads below 2048)
 *                    it is the minimum chunk length: the blocks of all
 *                    sequences are cut into equal chunks of at least
 *                    partition_size tokens (C blocks, see the workspace
 *                    layout below), one wave per chunk and kv head, and a
 *                    chunk yields one record per sequence it reaches.  With
 *                    batch * kv_heads at or above 2048, record r of a row
 *                    covers exactly partition r.  Records hold (reference
 *                    max, sum, normalised output) and are merged by
 *                    log-sum-exp; the result does not depend on where the
 *                    splits fall, up to rounding.
 *   workspace        device buffer of >= pa_decode_workspace_size bytes
 *                    (may be NULL when that is 0); not shared by
 *                    concurrent calls
 * L_b = 0 gives a zero output row and lse = -inf.  fp32 accumulation,
 * output rounded to fp16 to nearest even.  K/V are loaded with the
 * non-temporal cache policy (each block is read once per call); tables that
 * alias blocks across sequences (a shared prefix) are served faster by
 * pa_decode_shared_prefix.
 */
int pa_decode(void* out, float* lse_out, const void* q, const void* k_pool,
              const void* v_pool, const int32_t* block_table, int max_blocks,
              const int32_t* context_lens, int max_context_len, int batch, int q_heads,
              int kv_heads, int head_dim, int block_size, int num_blocks, float scale,
              int partition_size, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode over an int8 cache with fp32 per-(token, kv head) scales: the
 * cached value is code * scale ([KV-OPT] "三、实现示例" dequantize), folded
 * into the score (scale_k) and the softmax weight (scale_v) in fp32.
 */
int pa_decode_int8(void* out, float* lse_out, const void* q, const int8_t* k_pool,
                   const int8_t* v_pool, const float* k_scale, const float* v_scale,
                   const int32_t* block_table, int max_blocks, const int32_t* context_lens,
                   int max_context_len, int batch, int q_heads, int kv_heads, int head_dim,
                   int block_size, int num_blocks, float scale, int partition_size,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode over an FP8 (OCP E4M3) cache with fp32 per-(token, kv head)
 * scales (see pa_write_kv_fp8): codes become exact fp16 values on the way
 * in; the scales enter as for pa_decode_int8.
 */
int pa_decode_fp8(void* out, float* lse_out, const void* q, const uint8_t* k_pool,
                  const uint8_t* v_pool, const float* k_scale, const float* v_scale,
                  const int32_t* block_table, int max_blocks, const int32_t* context_lens,
                  int max_context_len, int batch, int q_heads, int kv_heads, int head_dim,
                  int block_size, int num_blocks, float scale, int partition_size,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  Same arguments, results and status
 * codes as pa_decode (fp16 caches), minus workspace / workspace_bytes; the
 * same kernels run.  The split-K records go to a device array inside the
 * library (one per device, PA_NOALLOC_SCRATCH_BYTES, held from the first
 * call on that device until the process ends).  Nothing is allocated: no
 * hipMalloc, no hipFree, no allocating library routine.
 *   - Shapes whose records need more than PA_NOALLOC_SCRATCH_BYTES
 *     (pa_decode_workspace_size with the same arguments) return
 *     PA_ERR_WORKSPACE before anything touches the device.
 *   - Every call on one device shares that device's array, which keeps the
 *     last call's records: calls that overlap on one device (concurrent
 *     streams, or threads) race and must be serialised by the caller.
 *     Calls on one stream are ordered and safe.
 *   - The first call on each device looks up the array's device address
 *     (PA_ERR_HIP if that fails, e.g. no device).
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int pa_decode_noalloc(void* out, float* lse_out, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_table, int max_blocks,
                      const int32_t* context_lens, int max_context_len, int batch, int q_heads,
                      int kv_heads, int head_dim, int block_size, int num_blocks, float scale,
                      int partition_size, void* stream);

/*
 * One decode step with the KV write folded in: writes each sequence's new
 * token (k_new / v_new, fp16 [batch, kv_heads, head_dim], the token at
 * position L_b - 1, L_b = context_lens[b] including it) into the slot the
 * block table gives for that position - copied for fp16 caches, quantised
 * per (token, kv head) row for int8 and FP8 exactly as pa_write_kv_int8 /
 * pa_write_kv_fp8 do - and computes out / lse_out as pa_decode would
 * afterwards.  Equivalent to pa_write_kv* with slot_mapping[b] =
 * block_table[b][(L_b - 1) / 16] * 16 + (L_b - 1) % 16, then pa_decode*
 * (WriteKV then page-table attention, [ATB-PA] "踩坑三" and "PagedAttention
 * 的 Attention 计算修改").  Two launches on `stream`: the partition kernel
 * over tokens [0, L_b - 1), whose extra workgroups do the write and the new
 * token's (max, sum, output) record, then the log-sum-exp merge of both
 * record sets; the write thus overlaps the attention instead of preceding
 * it.  The split is always taken (never the one-launch direct path).
 *   workspace  >= pa_decode_append_workspace_size(...) bytes: the
 *              pa_decode_partials layout, then 256-byte aligned float2
 *              (m, l) [batch][q_heads] and fp16 u [batch][q_heads][head_dim]
 *              for the new tokens
 *   k_scale / v_scale (8-bit caches)  fp32 [num_blocks, kv_heads, 16],
 *              read and written
 * L_b = 0 gives a zero row and writes nothing for b; L_b outside
 * [0, max_context_len] gives a NaN row; a table entry for position L_b - 1
 * outside the pool skips b's write and gives NaN rows.  Other arguments,
 * status codes and caller contracts as pa_decode; additionally each new
 * token's slot must lie in a block no other sequence of the call uses.
 */
size_t pa_decode_append_workspace_size(int batch, int q_heads, int kv_heads, int head_dim,
                                       int max_context_len, int partition_size);

int pa_decode_append(void* out, float* lse_out, const void* q, const void* k_new,
                     const void* v_new, void* k_pool, void* v_pool, const int32_t* block_table,
                     int max_blocks, const int32_t* context_lens, int max_context_len, int batch,
                     int q_heads, int kv_heads, int head_dim, int block_size, int num_blocks,
                     float scale, int partition_size, void* workspace, size_t workspace_bytes,
                     void* stream);

int pa_decode_append_int8(void* out, float* lse_out, const void* q, const void* k_new,
                          const void* v_new, int8_t* k_pool, int8_t* v_pool, float* k_scale,
                          float* v_scale, const int32_t* block_table, int max_blocks,
                          const int32_t* context_lens, int max_context_len, int batch,
                          int q_heads, int kv_heads, int head_dim, int block_size,
                          int num_blocks, float scale, int partition_size, void* workspace,
                          size_t workspace_bytes, void* stream);

int pa_decode_append_fp8(void* out, float* lse_out, const void* q, const void* k_new,
                         const void* v_new, uint8_t* k_pool, uint8_t* v_pool, float* k_scale,
                         float* v_scale, const int32_t* block_table, int max_blocks,
                         const int32_t* context_lens, int max_context_len, int batch,
                         int q_heads, int kv_heads, int head_dim, int block_size,
                         int num_blocks, float scale, int partition_size, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * The two stages pa_decode runs, exported for callers that combine
 * partial results from several sources (for example one sequence's
 * context split across devices, or a shared prefix attended once and
 * merged with each private suffix).
 *
 * pa_decode_partials / pa_decode_partials_int8 / pa_decode_partials_fp8:
 * same arguments as pa_decode / pa_decode_int8 / pa_decode_fp8 without out
 * and lse_out; always write the
 * partition records into the workspace, which must hold
 * pa_decode_workspace_size(..., partition_size resolved, ...) bytes
 * computed with max_context_len > partition_size, i.e. room for
 * n_part + 1 records per (b, h), n_part = ceil(max_context_len / P).
 * Workspace layout (P = resolved partition size):
 *   int32  header[64 + batch]           header[0] = record mode:
 *                                       1 when batch * kv_heads >= 2048:
 *                                         record r covers partition r,
 *                                         tokens [rP, min((r+1)P, L_b));
 *                                       0 otherwise (balanced chunks): the
 *                                         blocks of all sequences, laid end
 *                                         to end in batch order (sequence b
 *                                         owns blocks [F_b, F_b + nb_b),
 *                                         nb_b = ceil(L_b / 16), 0 for an
 *                                         empty or invalid length), are cut
 *                                         into chunks of C = max(P / 16,
 *                                         ceil(T / floor(2048 / kv_heads)))
 *                                         blocks, T = sum nb_b; record r of
 *                                         b covers b's blocks in chunk
 *                                         floor(F_b / C) + r, and
 *                                         header[64 + b] holds b's record
 *                                         count (written for L_b > 0 only).
 *                                       One wave streams a chunk's blocks
 *                                       for one kv head and merges them
 *                                       online, one record per sequence.
 *                                       The header takes 256-byte units.
 *   float2 ml[n_part+1][batch][q_heads] (m, l), record-major (slot r of
 *                                       every (b, h) row together): m = a
 *                                       reference point in
 *                                       log2 units, at most the record's
 *                                       largest score s = scale * log2(e) *
 *                                       q.k (and within 8 of it); l = sum of
 *                                       2^(s - m); m + log2(l) is the
 *                                       record's log-sum-exp
 *                                       (256-byte aligned after the header)
 *   fp16   u[n_part+1][batch][q_heads][head_dim]  normalised output of the
 *                                       record, sum 2^(s-m) v / l, rounded
 *                                       to nearest even (a convex
 *                                       combination of V rows, so within
 *                                       V's range); 256-byte aligned after ml
 * Records past a row's count are not written.
 *
 * pa_merge_partials: out[b,h] = sum_r w_r u_r / sum_r w_r with
 * w_r = 2^(m_r - M) l_r over the row's records, M = max m_r, accumulated in
 * fp32; lse = ln 2 * (M + log2(sum_r w_r)).
 */
int pa_decode_partials(const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_table, int max_blocks,
                       const int32_t* context_lens, int max_context_len, int batch,
                       int q_heads, int kv_heads, int head_dim, int block_size,
                       int num_blocks, float scale, int partition_size, void* workspace,
                       size_t workspace_bytes, void* stream);

int pa_decode_partials_int8(const void* q, const int8_t* k_pool, const int8_t* v_pool,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_table, int max_blocks,
                            const int32_t* context_lens, int max_context_len, int batch,
                            int q_heads, int kv_heads, int head_dim, int block_size,
                            int num_blocks, float scale, int partition_size,
                            void* workspace, size_t workspace_bytes, void* stream);

int pa_decode_partials_fp8(const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_table, int max_blocks,
                           const int32_t* context_lens, int max_context_len, int batch,
                           int q_heads, int kv_heads, int head_dim, int block_size,
                           int num_blocks, float scale, int partition_size,
                           void* workspace, size_t workspace_bytes, void* stream);

int pa_merge_partials(void* out, float* lse_out, const int32_t* context_lens,
                      int max_context_len, int batch, int q_heads, int head_dim,
                      int partition_size, const void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Shared-prefix decode.  The adg.csdn.net article on ATB's KV Cache
 * management (section "Prefix Caching") keeps one copy of the KV of a
 * prefix common to many requests (a system prompt), and the zskr.cn article
 * on ATB's PagedAttention (section "踩坑二") has those pages referenced by
 * every request that shares them.  pa_decode reads such a page once per
 * referencing sequence; these entry points read each shared page once per
 * kv head for all sequences together: the queries of all sequences (for kv
 * head g, the G query heads of every sequence) form 16-query tiles against
 * the shared keys on the matrix cores, giving one (max, sum, output) record
 * per (sequence, query head, prefix partition) - partitions of 16 to 256
 * tokens, sized so that the prefix work runs about 512 waves; the private
 * suffixes [prefix_len, L_b) are decoded as by pa_decode_partials; one
 * log-sum-exp merge combines both record sets.  The result is the same
 * attention as pa_decode (up to rounding order).
 *
 *   prefix_len       tokens of the shared prefix: a positive multiple of 16,
 *                    at most max_context_len.
 *   block_table      as for pa_decode; caller contract: for every b,
 *                    block_table[b][j] == block_table[0][j] for
 *                    j < prefix_len / 16 (the prefix ids are read from row
 *                    0 only) and context_lens[b] >= prefix_len.  A sequence
 *                    with context_lens[b] < prefix_len or > max_context_len
 *                    gets NaN rows.
 *   workspace        pa_decode_shared_prefix_workspace_size(...) bytes,
 *                    required (the split always runs).
 *   all other arguments as for pa_decode / pa_decode_int8 / pa_decode_fp8;
 *   the suffixes are split into at most four partitions of 16 to 256
 *   tokens (by the longest suffix, max_context_len - prefix_len), and the
 *   suffix work is cut into balanced chunks of at most one partition.
 *
 * Returns PA_ERR_SHAPE for a bad prefix_len, otherwise the codes of
 * pa_decode.  Launches, in order on `stream`: one kernel holding both the
 * prefix work and the suffix partition work (independent record sets), then
 * the merge kernel.
 */
size_t pa_decode_shared_prefix_workspace_size(int batch, int q_heads, int kv_heads,
                                              int head_dim, int max_context_len,
                                              int prefix_len);

int pa_decode_shared_prefix(void* out, float* lse_out, const void* q, const void* k_pool,
                            const void* v_pool, const int32_t* block_table, int max_blocks,
                            const int32_t* context_lens, int max_context_len, int batch,
                            int q_heads, int kv_heads, int head_dim, int block_size,
                            int num_blocks, float scale, int prefix_len, void* workspace,
                            size_t workspace_bytes, void* stream);

int pa_decode_shared_prefix_int8(void* out, float* lse_out, const void* q, const int8_t* k_pool,
                                 const int8_t* v_pool, const float* k_scale,
                                 const float* v_scale, const int32_t* block_table,
                                 int max_blocks, const int32_t* context_lens,
                                 int max_context_len, int batch, int q_heads, int kv_heads,
                                 int head_dim, int block_size, int num_blocks, float scale,
                                 int prefix_len, void* workspace, size_t workspace_bytes,
                                 void* stream);

int pa_decode_shared_prefix_fp8(void* out, float* lse_out, const void* q, const uint8_t* k_pool,
                                const uint8_t* v_pool, const float* k_scale,
                                const float* v_scale, const int32_t* block_table,
                                int max_blocks, const int32_t* context_lens,
                                int max_context_len, int batch, int q_heads, int kv_heads,
                                int head_dim, int block_size, int num_blocks, float scale,
                                int prefix_len, void* workspace, size_t workspace_bytes,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
