// Block copy for copy-on-write: whole physical blocks of the K and V pools
// (and, for 8-bit pools, their per-token scales) are copied src -> dst.
//
// The zskr.cn article on ATB's PagedAttention ("踩坑三") updates a page that
// several requests share by copy-on-write: a fresh page is taken, the old
// page's contents copied into it, and only then is the new token written.
// This is that copy for a batch of (src, dst) pairs, done on the device so
// the pools never leave HBM.  Pool layout [num_blocks, 16, kv_heads,
// head_dim] makes a block one contiguous run of 16 * kv_heads * head_dim
// elements; scales [num_blocks, kv_heads, 16] make a block's scales one run
// of kv_heads * 16 floats.
//
// Grid: x = pair, y = 16 KiB chunk of the block; 16-byte vector copies.
// Pairs naming a block outside [0, num_blocks) are skipped.
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kChunkBytes = kThreads * 16 * 4;   // 16 KiB per workgroup

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(const CopyParams p) {
  const int pair = blockIdx.x;
  const int src = p.pairs[2 * pair], dst = p.pairs[2 * pair + 1];
  if ((unsigned)src >= (unsigned)p.num_blocks || (unsigned)dst >= (unsigned)p.num_blocks) return;
  const size_t chunks = p.block_bytes / 16;      // block_bytes is a multiple of 16
  const size_t c0 = (size_t)blockIdx.y * (kChunkBytes / 16);
  const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const char*>(p.k_pool) +
                                                   (size_t)src * p.block_bytes);
  const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const char*>(p.v_pool) +
                                                   (size_t)src * p.block_bytes);
  uint4* kd = reinterpret_cast<uint4*>(static_cast<char*>(p.k_pool) + (size_t)dst * p.block_bytes);
  uint4* vd = reinterpret_cast<uint4*>(static_cast<char*>(p.v_pool) + (size_t)dst * p.block_bytes);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const size_t i = c0 + (size_t)r * kThreads + threadIdx.x;
    if (i < chunks) {
      kd[i] = ks[i];
      vd[i] = vs[i];
    }
  }
  if (p.k_scale && blockIdx.y == 0) {
    const int n = p.scales_per_block;            // kv_heads * 16 floats
    for (int i = threadIdx.x; i < n; i += kThreads) {
      p.k_scale[(size_t)dst * n + i] = p.k_scale[(size_t)src * n + i];
      p.v_scale[(size_t)dst * n + i] = p.v_scale[(size_t)src * n + i];
    }
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t stream) {
  if (p.num_pairs == 0) return hipSuccess;
  const size_t chunks_per_block = (p.block_bytes + kChunkBytes - 1) / kChunkBytes;
  dim3 grid((unsigned)p.num_pairs, (unsigned)chunks_per_block);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
