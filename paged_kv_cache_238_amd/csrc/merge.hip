// Log-sum-exp merge of split-K partition records into the final fp16 row.
//
// Record r of sequence b, query head h carries (m_r, l_r, u_r) for one
// stretch of its blocks (a partition, or a balanced chunk's share of the
// sequence, as the workspace header says): a reference point m_r for its
// scores (log2 units), the sum l_r of 2^(s - m_r), and the normalised
// output u_r = sum 2^(s - m_r) v / l_r in fp16.  With M = max_r m_r and
// w_r = 2^(m_r - M) l_r:
//   out = sum_r w_r u_r / sum_r w_r,   lse = ln2 * (M + log2 sum_r w_r).
// This is the running-max rescaling of the zskr.cn article's PagedAttention
// kernel (section "PagedAttention 的 Attention 计算修改") applied once
// across partitions instead of token by token, followed by that kernel's
// final normalisation and fp16 store.
//
// Rows with at most 17 * 256 / D records (the record stride bounds them): one wave
// per (sequence, query head), four rows per workgroup; lanes are D/4 float4
// columns x 256/D record phases, every record a lane needs is loaded at
// once (one memory round trip), and the phases are added by shuffles in a
// fixed order.  Longer rows: one workgroup of 256 lanes per row, D/4
// columns x 1024/D phases, phases added through LDS in a fixed order.  Both
// are deterministic.
//
// Shared-prefix decode merges two record sets per row: the records over the
// private suffix [prefix, L) and n_pre records over the shared prefix;
// both enter the same sums (the log-sum-exp merge is associative).  The
// append path uses the second set for the newest token of each row (one
// record) and the first for tokens [0, L - 1).
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kHeld = 8;        // records per lane held in registers (one round trip)
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.693147180559945309f;

// Maximum over the workgroup, through LDS; every lane gets it.
__device__ __forceinline__ float block_max(float x, float* s_max) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = x;
  __syncthreads();
  x = s_max[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) x = fmaxf(x, s_max[i]);
  return x;
}

// Records the partition kernel wrote for a sequence of (valid) length L:
// one per partition, or the count its balanced chunks stored in the header.
__device__ __forceinline__ int suffix_records(const MergeParams& p, int b, int L) {
  if (L == 0) return 0;
  // (a count is at most rec_stride when the partition kernel wrote it; the
  // clamp keeps any other header within the row's record slots)
  if (p.header[0] == 0) return min(max(p.header[kCountsAt + b], 0), p.rec_stride);
  return (L + p.partition_size - 1) / p.partition_size;
}

// Adds record (m, l, u) with weight w = 2^(m - M) * l: u holds four fp16
// values of the record's normalised output, so its unnormalised sum is w * u
// against the common reference M.
__device__ __forceinline__ void accumulate(float2 ml, uint2 u, float Mu, float4& acc, float& den) {
  typedef _Float16 h2v __attribute__((ext_vector_type(2)));
  const float wgt = __builtin_amdgcn_exp2f(ml.x - Mu) * ml.y;
  const h2v a = __builtin_bit_cast(h2v, u.x), c = __builtin_bit_cast(h2v, u.y);
  den += wgt;
  acc.x = fmaf(wgt, (float)a[0], acc.x);
  acc.y = fmaf(wgt, (float)a[1], acc.y);
  acc.z = fmaf(wgt, (float)c[0], acc.z);
  acc.w = fmaf(wgt, (float)c[1], acc.w);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}

template <int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(const MergeParams p) {
  constexpr int COLS = D / 4;              // float4 columns
  constexpr int PH = kThreads / COLS;      // partition phases
  __shared__ float4 s_acc[PH][COLS];
  __shared__ float s_den[PH];
  __shared__ float s_max[kThreads / 64];

  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, col = tid % COLS, ph = tid / COLS;
  const size_t row = (size_t)b * p.q_heads + h;
  const int L = p.context_lens[b] - p.token_offset;

  if (L < 0 || L > p.max_context_len) {
    for (int d = tid; d < D; d += kThreads) p.out[row * D + d] = 0x7E00;
    if (tid == 0 && p.lse) p.lse[row] = __builtin_nanf("");
    return;
  }
  // Append mode: the row's last token is its own record in the second set;
  // a sequence with no tokens has neither.
  const int n_suf = L > 0 ? suffix_records(p, b, L - p.len_trim) : 0;
  const int n_pre = (p.pre_ml && (L > 0 || !p.len_trim)) ? p.n_pre : 0;
  const int n = n_suf + n_pre;               // records: suffix, then prefix
  if (n == 0) {
    for (int d = tid; d < D; d += kThreads) p.out[row * D + d] = 0;
    if (tid == 0 && p.lse) p.lse[row] = kNegInf;
    return;
  }
  // Record-major sets: record i of this row sits i * rows entries in.
  const size_t rows = (size_t)p.batch * p.q_heads;
  const float2* ml = p.part_ml + row;
  const uint2* o = reinterpret_cast<const uint2*>(p.part_o + row * D);
  const float2* ml2 = n_pre ? p.pre_ml + row : nullptr;
  const uint2* o2 = n_pre ? reinterpret_cast<const uint2*>(p.pre_o + row * D) : nullptr;
  auto rec_ml = [&](int i) { return i < n_suf ? ml[i * rows] : ml2[(i - n_suf) * rows]; };
  auto rec_o = [&](int i) {
    return i < n_suf ? o[(size_t)i * rows * COLS + col] : o2[(size_t)(i - n_suf) * rows * COLS + col];
  };

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  float M = kNegInf;
  if (n <= PH * kHeld) {
    // Every record this lane needs (phase ph: records ph, ph + PH, ...) is
    // loaded at once, so the whole merge costs one memory round trip.
    float2 r[kHeld];
    uint2 v[kHeld];
#pragma unroll
    for (int k = 0; k < kHeld; ++k) {
      const int i = ph + k * PH;
      r[k] = make_float2(kNegInf, 0.f);
      v[k] = make_uint2(0, 0);
      if (i < n) {
        r[k] = rec_ml(i);
        v[k] = rec_o(i);
      }
    }
#pragma unroll
    for (int k = 0; k < kHeld; ++k) M = fmaxf(M, r[k].x);
    M = block_max(M, s_max);
    const float Mu = (M == kNegInf) ? 0.f : M;
#pragma unroll
    for (int k = 0; k < kHeld; ++k) {
      if (ph + k * PH < n) accumulate(r[k], v[k], Mu, acc, den);
    }
  } else {
    for (int i = tid; i < n; i += kThreads) M = fmaxf(M, rec_ml(i).x);
    M = block_max(M, s_max);
    const float Mu = (M == kNegInf) ? 0.f : M;
    for (int i = ph; i < n; i += PH) accumulate(rec_ml(i), rec_o(i), Mu, acc, den);
  }
  s_acc[ph][col] = acc;
  if (col == 0) s_den[ph] = den;
  __syncthreads();
  if (ph == 0) {
    float dsum = 0.f;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < PH; ++k) {
      dsum += s_den[k];
      const float4 v = s_acc[k][col];
      a.x += v.x;
      a.y += v.y;
      a.z += v.z;
      a.w += v.w;
    }
    uint16_t* dst = p.out + row * D + col * 4;
    dst[0] = f32_to_f16_bits(a.x / dsum);
    dst[1] = f32_to_f16_bits(a.y / dsum);
    dst[2] = f32_to_f16_bits(a.z / dsum);
    dst[3] = f32_to_f16_bits(a.w / dsum);
    if (col == 0 && p.lse) p.lse[row] = (M + log2f(dsum)) * kLn2;
  }
}

constexpr int kWaveHeld = 17;   // records per lane in the wave-per-row kernel (34 at D = 128:
                                // n_part + 1 records for 32 partitions)
constexpr int kRowsPerGroup = kThreads / 64;

template <int D>
__global__ __launch_bounds__(kThreads) void merge_wave_kernel(const MergeParams p) {
  constexpr int COLS = D / 4;              // float4 columns
  constexpr int PH = 64 / COLS;            // record phases within the wave
  const int lane = threadIdx.x & 63, col = lane % COLS, ph = lane / COLS;
  const long long rowid = (long long)blockIdx.x * kRowsPerGroup + (threadIdx.x >> 6);
  if (rowid >= (long long)p.batch * p.q_heads) return;
  const int b = (int)(rowid / p.q_heads);
  const size_t row = (size_t)rowid;
  // The length and the record mode and count in one round trip (the
  // header always holds a count slot per sequence).
  const int L = p.context_lens[b] - p.token_offset;
  const int rec_mode = p.header[0];
  const int rec_count = min(max(p.header[kCountsAt + b], 0), p.rec_stride);
  if (L < 0 || L > p.max_context_len) {
    for (int d = lane; d < D; d += 64) p.out[row * D + d] = 0x7E00;
    if (lane == 0 && p.lse) p.lse[row] = __builtin_nanf("");
    return;
  }
  // Append mode: the row's last token is its own record in the second set;
  // a sequence with no tokens has neither.
  const int Ls = L > 0 ? L - p.len_trim : 0;
  const int n_suf = Ls == 0 ? 0 : rec_mode == 0 ? rec_count : (Ls + p.partition_size - 1) / p.partition_size;
  const int n_pre = (p.pre_ml && (L > 0 || !p.len_trim)) ? p.n_pre : 0;
  const int n = n_suf + n_pre;
  if (n == 0) {
    for (int d = lane; d < D; d += 64) p.out[row * D + d] = 0;
    if (lane == 0 && p.lse) p.lse[row] = kNegInf;
    return;
  }
  // Record-major sets: record i of this row sits i * rows entries in.
  const size_t rows = (size_t)p.batch * p.q_heads;
  const float2* ml = p.part_ml + row;
  const uint2* o = reinterpret_cast<const uint2*>(p.part_o + row * D);
  const float2* ml2 = n_pre ? p.pre_ml + row : nullptr;
  const uint2* o2 = n_pre ? reinterpret_cast<const uint2*>(p.pre_o + row * D) : nullptr;
  float2 r[kWaveHeld];
  uint2 v[kWaveHeld];
#pragma unroll
  for (int k = 0; k < kWaveHeld; ++k) {
    const int i = ph + k * PH;
    r[k] = make_float2(kNegInf, 0.f);
    v[k] = make_uint2(0, 0);
    if (i < n) {
      r[k] = i < n_suf ? ml[i * rows] : ml2[(i - n_suf) * rows];
      v[k] = i < n_suf ? o[(size_t)i * rows * COLS + col]
                       : o2[(size_t)(i - n_suf) * rows * COLS + col];
    }
  }
  float M = kNegInf;
#pragma unroll
  for (int k = 0; k < kWaveHeld; ++k) M = fmaxf(M, r[k].x);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float Mu = (M == kNegInf) ? 0.f : M;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
#pragma unroll
  for (int k = 0; k < kWaveHeld; ++k) {
    if (ph + k * PH < n) accumulate(r[k], v[k], Mu, acc, den);
  }
  // phases in order: lane col of phase q holds its partial sums
  float dsum = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int q = 0; q < PH; ++q) {
    const int src = col + q * COLS;
    dsum += __shfl(den, src);
    a.x += __shfl(acc.x, src);
    a.y += __shfl(acc.y, src);
    a.z += __shfl(acc.z, src);
    a.w += __shfl(acc.w, src);
  }
  if (ph == 0) {
    uint16_t* dst = p.out + row * D + col * 4;
    dst[0] = f32_to_f16_bits(a.x / dsum);
    dst[1] = f32_to_f16_bits(a.y / dsum);
    dst[2] = f32_to_f16_bits(a.z / dsum);
    dst[3] = f32_to_f16_bits(a.w / dsum);
    if (col == 0 && p.lse) p.lse[row] = (M + log2f(dsum)) * kLn2;
  }
}

template <int D>
hipError_t launch_d(const MergeParams& p, hipStream_t stream) {
  // records per row are at most rec_stride (+ the prefix records)
  if (p.rec_stride + (p.pre_ml ? p.n_pre : 0) <= kWaveHeld * (256 / D)) {
    const long long rows = (long long)p.batch * p.q_heads;
    const unsigned groups = (unsigned)((rows + kRowsPerGroup - 1) / kRowsPerGroup);
    hipLaunchKernelGGL(merge_wave_kernel<D>, dim3(groups), dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(merge_kernel<D>, dim3(p.q_heads, p.batch), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  if (p.head_dim == 128) return launch_d<128>(p, stream);
  if (p.head_dim == 64) return launch_d<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
