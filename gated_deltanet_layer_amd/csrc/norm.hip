// norm.hip -- gated RMSNorm: y = o / sqrt(mean(o^2) + eps) * w * silu(z)
// per row of 128 values (one row per token and V-head).
//
// Method: the xwen CLAUDE.md page, section "Architecture cheat sheet", gated
// DeltaNet paragraph (norm, times ssm_norm.weight [128], then times silu(z));
// the weight is used as stored (section "GGUF facts that differ from the HF
// checkpoint": norm weights arrive multiply-ready).
//
// 16 lanes per row with 16-byte accesses; HBM-bound: reads o and z, writes
// y (3 x 128 act values per row).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kNormThreads = 256;
constexpr int kLanesPerRow = 16;             // 8 values per lane
constexpr int kRowsPerBlock = kNormThreads / kLanesPerRow;
constexpr int kRowsPerThread = 1;

// 8 consecutive activation values <-> two float4.
__device__ __forceinline__ void load8(const float *p, size_t i, float4 &a, float4 &b) {
  a = *reinterpret_cast<const float4 *>(p + i);
  b = *reinterpret_cast<const float4 *>(p + i + 4);
}
__device__ __forceinline__ void load8(const bf16_t *p, size_t i, float4 &a, float4 &b) {
  const uint4 w = *reinterpret_cast<const uint4 *>(p + i);
  a = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                  __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
  b = make_float4(__uint_as_float(w.z << 16), __uint_as_float(w.z & 0xffff0000u),
                  __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xffff0000u));
}
__device__ __forceinline__ void store8(float *p, size_t i, float4 a, float4 b) {
  *reinterpret_cast<float4 *>(p + i) = a;
  *reinterpret_cast<float4 *>(p + i + 4) = b;
}
__device__ __forceinline__ void store8(bf16_t *p, size_t i, float4 a, float4 b) {
  uint4 w;
  w.x = static_cast<uint32_t>(f32_to_bf16(a.x)) | (static_cast<uint32_t>(f32_to_bf16(a.y)) << 16);
  w.y = static_cast<uint32_t>(f32_to_bf16(a.z)) | (static_cast<uint32_t>(f32_to_bf16(a.w)) << 16);
  w.z = static_cast<uint32_t>(f32_to_bf16(b.x)) | (static_cast<uint32_t>(f32_to_bf16(b.y)) << 16);
  w.w = static_cast<uint32_t>(f32_to_bf16(b.z)) | (static_cast<uint32_t>(f32_to_bf16(b.w)) << 16);
  *reinterpret_cast<uint4 *>(p + i) = w;
}

// 16 lanes per row, 8 values per lane (16-byte bf16 or 32-byte fp32 accesses),
// 4 rows per wave at a time; each thread handles kRowsPerThread rows that
// lie kRowsPerBlock apart, all loaded before any is used.
// kConv: blocks past the norm's also write the new conv states of the
// packed sequences (conv_state_pair, 2 channels per thread), in the same
// launch: both only read what earlier kernels left.
template <typename TA, bool kConv>
__global__ __launch_bounds__(kNormThreads) void norm_kernel(NormParams p, ConvStateParams cp, int norm_blocks,
                                                            int conv_per_seq) {
  if (kConv && static_cast<int>(blockIdx.x) >= norm_blocks) {
    const int b = blockIdx.x - norm_blocks;
    conv_state_pair<TA>(cp, b / conv_per_seq, 2 * ((b % conv_per_seq) * kNormThreads + threadIdx.x));
    return;
  }
  const int sub = threadIdx.x % kLanesPerRow;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock * kRowsPerThread + threadIdx.x / kLanesPerRow;
  const float4 w0 = *reinterpret_cast<const float4 *>(p.w + 8 * sub);
  const float4 w1 = *reinterpret_cast<const float4 *>(p.w + 8 * sub + 4);
  float4 o0[kRowsPerThread], o1[kRowsPerThread], z0[kRowsPerThread], z1[kRowsPerThread];
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int64_t row = min(row0 + u * kRowsPerBlock, p.n_rows - 1);
    const size_t i = static_cast<size_t>(row) * kHeadDim + 8 * sub;
    load8(static_cast<const TA *>(p.o), i, o0[u], o1[u]);
    load8(static_cast<const TA *>(p.z), i, z0[u], z1[u]);
  }
  static_assert(kLanesPerRow == 16, "one row per 16-lane DPP row");
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int64_t row = row0 + u * kRowsPerBlock;
    float ss = o0[u].x * o0[u].x + o0[u].y * o0[u].y + o0[u].z * o0[u].z + o0[u].w * o0[u].w +
               o1[u].x * o1[u].x + o1[u].y * o1[u].y + o1[u].z * o1[u].z + o1[u].w * o1[u].w;
    ss = row16_sum(ss);
    const float inv = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + p.eps);
    float4 y0, y1;
    y0.x = o0[u].x * inv * w0.x * siluf_(z0[u].x);
    y0.y = o0[u].y * inv * w0.y * siluf_(z0[u].y);
    y0.z = o0[u].z * inv * w0.z * siluf_(z0[u].z);
    y0.w = o0[u].w * inv * w0.w * siluf_(z0[u].w);
    y1.x = o1[u].x * inv * w1.x * siluf_(z1[u].x);
    y1.y = o1[u].y * inv * w1.y * siluf_(z1[u].y);
    y1.z = o1[u].z * inv * w1.z * siluf_(z1[u].z);
    y1.w = o1[u].w * inv * w1.w * siluf_(z1[u].w);
    if (row < p.n_rows) store8(static_cast<TA *>(p.y), static_cast<size_t>(row) * kHeadDim + 8 * sub, y0, y1);
  }
}

}  // namespace

hipError_t launch_norm(const NormParams &p, gdn_dtype act, hipStream_t s) {
  const int64_t blocks = (p.n_rows + kRowsPerBlock * kRowsPerThread - 1) / (kRowsPerBlock * kRowsPerThread);
  const ConvStateParams none{};
  if (act == GDN_BF16)
    hipLaunchKernelGGL((norm_kernel<bf16_t, false>), dim3(static_cast<unsigned>(blocks)), dim3(kNormThreads), 0, s, p,
                       none, static_cast<int>(blocks), 1);
  else
    hipLaunchKernelGGL((norm_kernel<float, false>), dim3(static_cast<unsigned>(blocks)), dim3(kNormThreads), 0, s, p,
                       none, static_cast<int>(blocks), 1);
  return hipGetLastError();
}

hipError_t launch_norm_conv_state(const NormParams &p, const ConvStateParams &cp, gdn_dtype act, hipStream_t s) {
  const int64_t blocks = (p.n_rows + kRowsPerBlock * kRowsPerThread - 1) / (kRowsPerBlock * kRowsPerThread);
  const int per_seq = (cp.C / 2 + kNormThreads - 1) / kNormThreads;
  const int64_t total = blocks + static_cast<int64_t>(cp.n_seqs) * per_seq;
  if (total == 0) return hipSuccess;
  if (act == GDN_BF16)
    hipLaunchKernelGGL((norm_kernel<bf16_t, true>), dim3(static_cast<unsigned>(total)), dim3(kNormThreads), 0, s, p,
                       cp, static_cast<int>(blocks), per_seq);
  else
    hipLaunchKernelGGL((norm_kernel<float, true>), dim3(static_cast<unsigned>(total)), dim3(kNormThreads), 0, s, p,
                       cp, static_cast<int>(blocks), per_seq);
  return hipGetLastError();
}

}  // namespace gdn
