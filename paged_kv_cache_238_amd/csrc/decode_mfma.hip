// Paged-attention decode, matrix-core form (query-head groups of 4, 8 or 16): the kernel wrapper and its
// launchers.  The kernel body and its description are in decode_mfma.h.
#include "decode_mfma.h"

namespace pa {
namespace {

using namespace mfma;

// Matrix-core decode kernel: one launch's workgroups run mfma_body on their
// own index (the shared-prefix launch runs it on part of its grid).
template <int D, int G, int KV, bool PREFIX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(PA_MFMA_WAVES_PER_EU)))
void decode_mfma_kernel(const DecodeParams p) {
  mfma_body<D, G, KV, PREFIX>(p, (int)blockIdx.x);
}

// Waves (kv heads) per workgroup.  Long contexts (chunks of many blocks, all
// alike): eight, so one workgroup reads whole token rows of an 8-head cache.
// Otherwise four, which keeps workgroups small enough to pack CUs evenly
// when chunks are short or uneven.
int waves_per_group(const DecodeParams& p) {
  if (p.kv_heads % 8 == 0 && p.max_context_len >= kLongContext) return 8;
  return (p.kv_heads % 4 == 0) ? 4 : (p.kv_heads % 2 == 0) ? 2 : 1;
}

template <int D, int G, int KV>
hipError_t launch_one(const DecodeParams& p, hipStream_t stream) {
  using Geo = Geometry<D, KV != kKvF16>;
  const int wpg = waves_per_group(p);
  const size_t lds = (size_t)wpg * kBlockTokens * Geo::kRowBytes + kIdCap * sizeof(int32_t);
  DecodeParams q = p;
  q.main_groups = (int)decode_workgroups(p, wpg);
  const unsigned grid = (unsigned)q.main_groups + append_workgroups(p, wpg);
  hipLaunchKernelGGL((decode_mfma_kernel<D, G, KV, false>), dim3(grid), dim3(64 * wpg), lds,
                     stream, q);
  return hipGetLastError();
}

template <int D, int KV>
hipError_t dispatch_group(const DecodeParams& p, hipStream_t stream) {
  switch (p.q_heads / p.kv_heads) {
    case 4: return launch_one<D, 4, KV>(p, stream);
    case 8: return launch_one<D, 8, KV>(p, stream);
    case 16: return launch_one<D, 16, KV>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t dispatch_format(const DecodeParams& p, int kv, hipStream_t stream) {
  switch (kv) {
    case kKvF16: return dispatch_group<D, kKvF16>(p, stream);
    case kKvI8: return dispatch_group<D, kKvI8>(p, stream);
    case kKvF8: return dispatch_group<D, kKvF8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, int kv, hipStream_t stream) {
  if (p.head_dim == 128) return dispatch_format<128>(p, kv, stream);
  if (p.head_dim == 64) return dispatch_format<64>(p, kv, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
