// Shared-prefix decode in one launch: the partition work over the private
// suffixes and the prefix work over the shared blocks are independent (they
// fill two record sets that the merge combines), so one grid holds both.
// Workgroups [0, prefix_groups) run the matrix-core prefix body, the rest
// the suffix body (VALU form for groups of 1 or 2, matrix-core form
// otherwise); the prefix workgroups come first so that they are dispatched
// before the suffix ones fill the GPU.  The prefix work, mostly served from cache, then overlaps the
// suffix streaming instead of following it.  Prefix caching: the adg.csdn.net
// article on ATB's KV Cache management, section "Prefix Caching"; each
// shared block is read once per kv head and query tile.
#include "decode_mfma.h"
#include "decode_valu.h"

namespace pa {
namespace {

constexpr int kFusedThreads = 256;   // at most four waves per workgroup

// Three waves per SIMD (<= 168 registers), which the matrix-core body is
// tuned for and the VALU body fits.
template <int D, int G, int KV>
__global__ __launch_bounds__(kFusedThreads)
__attribute__((amdgpu_waves_per_eu(PA_MFMA_WAVES_PER_EU)))
void shared_prefix_kernel(const DecodeParams ps, const DecodeParams pp, int prefix_groups) {
  const int wg = (int)blockIdx.x;
  if (wg < prefix_groups) {
    mfma::mfma_body<D, 16, KV, true>(pp, wg);
  } else if constexpr (G <= 2) {
    valu::valu_body<D, G, KV, false>(ps, wg - prefix_groups);
  } else {
    mfma::mfma_body<D, G, KV, false>(ps, wg - prefix_groups);
  }
}

template <int D, int G, int KV>
hipError_t launch_fused(const DecodeParams& ps, const DecodeParams& pp, hipStream_t stream) {
  using Geo = mfma::Geometry<D, KV != kKvF16>;
  const int wpg = (ps.kv_heads % 4 == 0) ? 4 : (ps.kv_heads % 2 == 0) ? 2 : 1;
  const unsigned suffix = decode_workgroups(ps, wpg);
  // Prefix workgroups: (tile group, partition, kv head) items, the waves
  // taking wpg consecutive query tiles, when there are at least wpg tiles:
  // the waves of a workgroup then load the same K/V lines together, so the
  // lines come from HBM once per workgroup (on 64 sequences sharing a
  // 1024-token prefix the call went from 56.1-56.3 to 54.9-55.0 us, one box,
  // alternating builds; with the default cache policy instead of the
  // non-temporal one, 56.8-57.0 us).  Otherwise (query tile, partition,
  // head group) items, the waves taking wpg kv heads.
  DecodeParams q = pp;
  q.prefix_tile_waves = pp.prefix_tiles >= wpg ? 1 : 0;
  const unsigned prefix =
      q.prefix_tile_waves
          ? (unsigned)((long long)((pp.prefix_tiles + wpg - 1) / wpg) * pp.n_part * pp.kv_heads)
          : (unsigned)((long long)pp.prefix_tiles * pp.n_part * (pp.kv_heads / wpg));
  const size_t lds = (size_t)wpg * kBlockTokens * Geo::kRowBytes + mfma::kIdCap * sizeof(int32_t);
  hipLaunchKernelGGL((shared_prefix_kernel<D, G, KV>), dim3(suffix + prefix), dim3(64 * wpg), lds,
                     stream, ps, q, (int)prefix);
  return hipGetLastError();
}

template <int D, int KV>
hipError_t fused_group(const DecodeParams& ps, const DecodeParams& pp, hipStream_t stream) {
  switch (ps.q_heads / ps.kv_heads) {
    case 1: return launch_fused<D, 1, KV>(ps, pp, stream);
    case 2: return launch_fused<D, 2, KV>(ps, pp, stream);
    case 4: return launch_fused<D, 4, KV>(ps, pp, stream);
    case 8: return launch_fused<D, 8, KV>(ps, pp, stream);
    case 16: return launch_fused<D, 16, KV>(ps, pp, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t fused_format(const DecodeParams& ps, const DecodeParams& pp, int kv,
                        hipStream_t stream) {
  switch (kv) {
    case kKvF16: return fused_group<D, kKvF16>(ps, pp, stream);
    case kKvI8: return fused_group<D, kKvI8>(ps, pp, stream);
    case kKvF8: return fused_group<D, kKvF8>(ps, pp, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_shared_prefix(const DecodeParams& ps, const DecodeParams& pp, int kv,
                                hipStream_t stream) {
  if (ps.head_dim == 128) return fused_format<128>(ps, pp, kv, stream);
  if (ps.head_dim == 64) return fused_format<64>(ps, pp, kv, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
