// norm.hip -- gated RMSNorm: y = o / sqrt(mean(o^2) + eps) * w * silu(z)
// per row of 128 values (one row per token and V-head).
//
// Method: the xwen CLAUDE.md page, section "Architecture cheat sheet", gated
// DeltaNet paragraph (norm, times ssm_norm.weight [128], then times silu(z));
// the weight is used as stored (section "GGUF facts that differ from the HF
// checkpoint": norm weights arrive multiply-ready).
//
// One wave per row, 2 values per lane; 4 rows per 256-thread block.
// HBM-bound: reads o and z, writes y (3 x 128 act values per row).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kNormThreads = 256;

template <typename TA>
__global__ __launch_bounds__(kNormThreads) void norm_kernel(NormParams p) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kNormThreads / kWave) + threadIdx.x / kWave;
  if (row >= p.n_rows) return;
  const int lane = lane_id();
  const size_t i = static_cast<size_t>(row) * kHeadDim + 2 * lane;
  const float2 o = Act<TA>::load2(static_cast<const TA *>(p.o), i);
  const float2 z = Act<TA>::load2(static_cast<const TA *>(p.z), i);
  const float2 w = *reinterpret_cast<const float2 *>(p.w + 2 * lane);
  const float ss = wave_sum(o.x * o.x + o.y * o.y);
  const float inv = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + p.eps);
  float2 y;
  y.x = o.x * inv * w.x * siluf_(z.x);
  y.y = o.y * inv * w.y * siluf_(z.y);
  Act<TA>::store2(static_cast<TA *>(p.y), i, y);
}

}  // namespace

hipError_t launch_norm(const NormParams &p, gdn_dtype act, hipStream_t s) {
  const int rows_per_block = kNormThreads / kWave;
  const int64_t blocks = (p.n_rows + rows_per_block - 1) / rows_per_block;
  if (act == GDN_BF16)
    hipLaunchKernelGGL(norm_kernel<bf16_t>, dim3(static_cast<unsigned>(blocks)), dim3(kNormThreads), 0, s, p);
  else
    hipLaunchKernelGGL(norm_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(kNormThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace gdn
