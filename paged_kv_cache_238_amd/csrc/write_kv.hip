// KV write ("reshape and cache"): each new token's K and V rows go to their
// slot in the paged pools.
//
// Pool layout [num_blocks, 16, kv_heads, head_dim] puts all kv heads of one
// slot next to each other, so a slot's K (or V) row is one contiguous run of
// kv_heads * head_dim elements, as is the new token's row in k_new / v_new.
// The fp16 write is therefore a 16-byte-vector row copy.  Semantics: the
// discosf.com article "KV Cache 优化与显存管理", section "三、实现示例",
// PhysicalPagePool.write_page (storage[page, kv, layer, offset] = data), and
// WriteKV in section "踩坑三" of the zskr.cn ATB PagedAttention article.
//
// The int8 and FP8 writes quantise each (token, kv head) row of head_dim
// values on the way in (per-row scale, quant.h).
#include "pa_internal.h"
#include "quant.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void write_kv_f16_kernel(const WriteParams p) {
  const int n16 = p.kv_heads * p.head_dim / 8;   // 16-byte chunks per row
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= n16) return;
  for (int tok = blockIdx.y; tok < p.num_tokens; tok += gridDim.y) {
    const int slot = p.slots[tok];
    if (slot < 0 || (long long)slot >= p.capacity) continue;
    const uint4* ks = reinterpret_cast<const uint4*>(p.k_new) + (size_t)tok * n16;
    const uint4* vs = reinterpret_cast<const uint4*>(p.v_new) + (size_t)tok * n16;
    uint4* kd = reinterpret_cast<uint4*>(p.k_pool) + (size_t)slot * n16;
    uint4* vd = reinterpret_cast<uint4*>(p.v_pool) + (size_t)slot * n16;
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

// One wave per (token, kv head) row; lane holds D/64 consecutive elements.
// FP8 = false: int8 codes; true: E4M3 codes.
template <int D, bool FP8>
__device__ __forceinline__ void quantise_row(const uint16_t* src, uint8_t* dst, float* scale_dst,
                                             int lane) {
  constexpr int PER = D / 64;
  float x[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    _Float16 h = __builtin_bit_cast(_Float16, src[lane * PER + e]);
    x[e] = (float)h;
  }
  uint8_t code[PER];
  const float s = quantise_vals<PER, FP8>(x, code);
#pragma unroll
  for (int e = 0; e < PER; ++e) dst[lane * PER + e] = code[e];
  if (lane == 0) *scale_dst = s;
}

template <int D, bool FP8>
__global__ __launch_bounds__(kThreads) void write_kv_q8_kernel(const WriteParams p) {
  const int lane = threadIdx.x & 63;
  const long long rowid = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (rowid >= (long long)p.num_tokens * p.kv_heads) return;
  const int tok = (int)(rowid / p.kv_heads), g = (int)(rowid % p.kv_heads);
  const int slot = p.slots[tok];
  if (slot < 0 || (long long)slot >= p.capacity) return;
  const size_t src = ((size_t)tok * p.kv_heads + g) * D;
  const size_t dst = ((size_t)slot * p.kv_heads + g) * D;
  const size_t sdst = ((size_t)(slot / 16) * p.kv_heads + g) * 16 + slot % 16;   // [NB, Hkv, 16]
  quantise_row<D, FP8>(p.k_new + src, static_cast<uint8_t*>(p.k_pool) + dst, p.k_scale + sdst,
                       lane);
  quantise_row<D, FP8>(p.v_new + src, static_cast<uint8_t*>(p.v_pool) + dst, p.v_scale + sdst,
                       lane);
}

}  // namespace

hipError_t launch_write_kv(const WriteParams& p, hipStream_t stream) {
  if (p.num_tokens == 0) return hipSuccess;
  const int n16 = p.kv_heads * p.head_dim / 8;
  dim3 grid((n16 + kThreads - 1) / kThreads, p.num_tokens < 65535 ? p.num_tokens : 65535);
  hipLaunchKernelGGL(write_kv_f16_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

namespace {

template <bool FP8>
hipError_t launch_q8(const WriteParams& p, hipStream_t stream) {
  if (p.num_tokens == 0) return hipSuccess;
  const long long rows = (long long)p.num_tokens * p.kv_heads;
  dim3 grid((unsigned)((rows + 3) / 4));
  if (p.head_dim == 128)
    hipLaunchKernelGGL((write_kv_q8_kernel<128, FP8>), grid, dim3(kThreads), 0, stream, p);
  else if (p.head_dim == 64)
    hipLaunchKernelGGL((write_kv_q8_kernel<64, FP8>), grid, dim3(kThreads), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_write_kv_int8(const WriteParams& p, hipStream_t stream) {
  return launch_q8<false>(p, stream);
}

hipError_t launch_write_kv_fp8(const WriteParams& p, hipStream_t stream) {
  return launch_q8<true>(p, stream);
}

}  // namespace pa
