// checks.hip -- state checkpoints and a non-finite guard around the mixer.
//
// Conv-state checkpoints: the conv state a later call needs to resume at
// token p of a sequence is the 3 raw qkv rows before p (the xwen CLAUDE.md
// page, section "Architecture cheat sheet": the conv state is the last 3
// columns of the fused qkv stream), copied bit for bit; rows before the
// sequence come from its incoming conv state. The delta-state checkpoints
// at the same tokens come from the chunked pass itself.
//
// Non-finite guard: one pass over a state buffer counting NaN/Inf values and
// taking max |x| over the finite ones (the serverAppConfigs commit-log page,
// the entry on gdn_hip state faults under prefix caching, records a GDN
// state checkpointed at a block boundary that went non-finite and was
// re-seeded from that page on every later turn). Results land in a device int32[2]
// the caller reads when it synchronises; a small kernel clears it first, so
// the pair can be captured in a HIP graph.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kCkptThreads = 256;

// One block per (sequence, checkpoint); 2 channels per thread and pass.
template <typename TA>
__global__ __launch_bounds__(kCkptThreads) void conv_ckpt_kernel(ConvCkptParams p) {
  const int n = blockIdx.x / p.cap;
  const int c = blockIdx.x % p.cap;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  if (seq0 < 0 || L < 0 || seq0 + L > p.n_tokens) return;
  const int64_t pos = static_cast<int64_t>(c + 1) * p.every;   // token index inside the sequence
  if (pos > L) return;
  const int C = kHeadDim * (2 * p.n_qk + p.n_v);
  const TA *qkv = static_cast<const TA *>(p.qkv);
  const TA *st = static_cast<const TA *>(p.st_in) + static_cast<size_t>(n) * (kConvK - 1) * C;
  TA *dst = static_cast<TA *>(p.ckpt) + (static_cast<size_t>(n) * p.cap + c) * (kConvK - 1) * C;
  for (int ch = 2 * threadIdx.x; ch < C; ch += 2 * kCkptThreads) {
#pragma unroll
    for (int r = 0; r < kConvK - 1; ++r) {
      const int64_t row = pos - (kConvK - 1) + r;              // row of [state; x], relative to token 0
      const float2 x = row < 0 ? Act<TA>::load2(st, static_cast<size_t>(kConvK - 1 + row) * C + ch)
                               : Act<TA>::load2(qkv, static_cast<size_t>(seq0 + row) * C + ch);
      Act<TA>::store2(dst, static_cast<size_t>(r) * C + ch, x);
    }
  }
}

__global__ void clear_stats_kernel(int32_t *stats) {
  if (threadIdx.x < 2) stats[threadIdx.x] = 0;
}

constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void state_check_kernel(const float *S, int64_t n, int32_t *stats) {
  int bad = 0;
  float mx = 0.f;
  const int64_t n4 = n / 4;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kCheckThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCheckThreads + threadIdx.x; i < n4; i += stride) {
    const float4 x = reinterpret_cast<const float4 *>(S)[i];
    const float v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (isfinite(v[e])) mx = fmaxf(mx, fabsf(v[e]));
      else ++bad;
    }
  }
  for (int64_t i = 4 * n4 + static_cast<int64_t>(blockIdx.x) * kCheckThreads + threadIdx.x; i < n; i += stride) {
    if (isfinite(S[i])) mx = fmaxf(mx, fabsf(S[i]));
    else ++bad;
  }
  // Wave reductions, then one atomic per wave (vector memory atomics).
  bad = wave_sum_i(bad);
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
  if (lane_id() == 0) {
    if (bad) atomicAdd(&stats[0], bad);
    // max |x| >= 0: the int order of the bit patterns is the float order.
    atomicMax(&stats[1], __float_as_int(mx));
  }
}

}  // namespace

hipError_t launch_conv_ckpt(const ConvCkptParams &p, gdn_dtype act, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(p.n_seqs) * p.cap));
  if (act == GDN_BF16)
    hipLaunchKernelGGL(conv_ckpt_kernel<bf16_t>, grid, dim3(kCkptThreads), 0, s, p);
  else
    hipLaunchKernelGGL(conv_ckpt_kernel<float>, grid, dim3(kCkptThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_state_check(const float *S, int64_t n_values, int32_t *stats, hipStream_t s) {
  hipLaunchKernelGGL(clear_stats_kernel, dim3(1), dim3(kWave), 0, s, stats);
  const int64_t want = (n_values / 4 + kCheckThreads - 1) / kCheckThreads;
  const unsigned blocks = static_cast<unsigned>(want < 1 ? 1 : (want > 2048 ? 2048 : want));
  hipLaunchKernelGGL(state_check_kernel, dim3(blocks), dim3(kCheckThreads), 0, s, S, n_values, stats);
  return hipGetLastError();
}

}  // namespace gdn
