// Paged-attention decode, VALU form (query-head groups of 1 or 2): the kernel wrapper and its
// launchers.  The kernel body and its description are in decode_valu.h.
#include "decode_valu.h"

namespace pa {
namespace {

using namespace valu;

// VALU decode kernel: one launch's workgroups run valu_body on their own
// index (the shared-prefix launch runs it on part of its grid).
template <int D, int G, int KV>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(const DecodeParams p) {
  valu_body<D, G, KV, true>(p, (int)blockIdx.x);
}

// Waves (kv heads) per workgroup: four when the heads divide evenly.
int waves_per_group(const DecodeParams& p) {
  return (p.kv_heads % 4 == 0) ? 4 : (p.kv_heads % 2 == 0) ? 2 : 1;
}

template <int D, int G, int KV>
hipError_t launch_one(const DecodeParams& p, hipStream_t stream) {
  const int wpg = waves_per_group(p);
  DecodeParams q = p;
  q.main_groups = (int)decode_workgroups(p, wpg);
  const unsigned grid = (unsigned)q.main_groups + append_workgroups(p, wpg);
  hipLaunchKernelGGL((decode_valu_kernel<D, G, KV>), dim3(grid), dim3(64 * wpg), 0, stream, q);
  return hipGetLastError();
}

template <int D, int KV>
hipError_t dispatch_group(const DecodeParams& p, hipStream_t stream) {
  switch (p.q_heads / p.kv_heads) {
    case 1: return launch_one<D, 1, KV>(p, stream);
    case 2: return launch_one<D, 2, KV>(p, stream);
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

hipError_t launch_decode_valu(const DecodeParams& p, int kv, hipStream_t stream) {
  if (p.head_dim == 128) return dispatch_format<128>(p, kv, stream);
  if (p.head_dim == 64) return dispatch_format<64>(p, kv, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, int kv, hipStream_t stream) {
  const int group = p.q_heads / p.kv_heads;
  if (group >= 4) return launch_decode_mfma(p, kv, stream);
  return launch_decode_valu(p, kv, stream);
}

}  // namespace pa
