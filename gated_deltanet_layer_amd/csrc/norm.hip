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
// 4 rows per wave, 16 rows per block.
template <typename TA>
__global__ __launch_bounds__(kNormThreads) void norm_kernel(NormParams p) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  if (row >= p.n_rows) return;
  const int sub = threadIdx.x % kLanesPerRow;
  const size_t i = static_cast<size_t>(row) * kHeadDim + 8 * sub;
  float4 o0, o1, z0, z1;
  load8(static_cast<const TA *>(p.o), i, o0, o1);
  load8(static_cast<const TA *>(p.z), i, z0, z1);
  const float4 w0 = *reinterpret_cast<const float4 *>(p.w + 8 * sub);
  const float4 w1 = *reinterpret_cast<const float4 *>(p.w + 8 * sub + 4);
  float ss = o0.x * o0.x + o0.y * o0.y + o0.z * o0.z + o0.w * o0.w +
             o1.x * o1.x + o1.y * o1.y + o1.z * o1.z + o1.w * o1.w;
  static_assert(kLanesPerRow == 16, "one row per 16-lane DPP row");
  ss = row16_sum(ss);
  const float inv = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + p.eps);
  float4 y0, y1;
  y0.x = o0.x * inv * w0.x * siluf_(z0.x);
  y0.y = o0.y * inv * w0.y * siluf_(z0.y);
  y0.z = o0.z * inv * w0.z * siluf_(z0.z);
  y0.w = o0.w * inv * w0.w * siluf_(z0.w);
  y1.x = o1.x * inv * w1.x * siluf_(z1.x);
  y1.y = o1.y * inv * w1.y * siluf_(z1.y);
  y1.z = o1.z * inv * w1.z * siluf_(z1.z);
  y1.w = o1.w * inv * w1.w * siluf_(z1.w);
  store8(static_cast<TA *>(p.y), i, y0, y1);
}

}  // namespace

hipError_t launch_norm(const NormParams &p, gdn_dtype act, hipStream_t s) {
  const int64_t blocks = (p.n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (act == GDN_BF16)
    hipLaunchKernelGGL(norm_kernel<bf16_t>, dim3(static_cast<unsigned>(blocks)), dim3(kNormThreads), 0, s, p);
  else
    hipLaunchKernelGGL(norm_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(kNormThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace gdn
