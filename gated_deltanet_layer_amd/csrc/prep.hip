// prep.hip -- causal depthwise conv (kernel 4, no bias) + SiLU + split +
// clamp-form L2 norm of q/k + beta/g gates, and the conv-state update.
//
// Method: the xwen CLAUDE.md page, section "Architecture cheat sheet", gated
// DeltaNet paragraph (conv over the whole fused width, SiLU over all of it,
// q | k | v split, x / max(||x||, eps), beta = sigmoid, g = ssm_a * softplus
// with ssm_a = -exp(A_log) per the section "GGUF facts that differ from the
// HF checkpoint").
//
// Grid: x = token tiles (kPrepTile tokens of one sequence; an empty sequence
// owns one tile that only moves its conv state), y = head block (128 fused
// channels: Hqk q heads, Hqk k heads, Hv v heads). One wave per block; each
// lane owns 2 adjacent channels and keeps the 3 previous raw rows in
// registers, so each qkv row is read once per tile (plus a 3-row halo).
// HBM-bound: per token it reads C act values and writes C fp32 values.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <typename TA>
__global__ __launch_bounds__(kWave) void prep_kernel(PrepParams p) {
  const int lane = lane_id();
  const int hb = blockIdx.y;
  int n, tile;
  if (!find_unit(p.cu, p.n_seqs, blockIdx.x, kPrepTile, 1, &n, &tile)) return;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  // Indices derived from cu_seqlens must stay inside the buffers.
  if (seq0 < 0 || L < 0 || seq0 + L > p.n_tokens) return;

  const int C = kHeadDim * (2 * p.n_qk + p.n_v);
  const int c = hb * kHeadDim + 2 * lane;
  const TA *qkv = static_cast<const TA *>(p.qkv);
  const TA *st_in = static_cast<const TA *>(p.st_in);
  TA *st_out = static_cast<TA *>(p.st_out);
  const size_t st_base = static_cast<size_t>(n) * (kConvK - 1) * C;

  const float4 w0 = reinterpret_cast<const float4 *>(p.conv_w)[c];
  const float4 w1 = reinterpret_cast<const float4 *>(p.conv_w)[c + 1];

  const int tau0 = tile * kPrepTile;
  const int ntok = min(kPrepTile, L - tau0);

  // Raw rows tau0-3 .. tau0-1 of [state; x]: the window before the tile.
  float2 xm[kConvK - 1];
#pragma unroll
  for (int r = 0; r < kConvK - 1; ++r) {
    const int pos = tau0 - (kConvK - 1) + r;
    xm[r] = pos < 0 ? Act<TA>::load2(st_in, st_base + static_cast<size_t>(pos + kConvK - 1) * C + c)
                    : Act<TA>::load2(qkv, static_cast<size_t>(seq0 + pos) * C + c);
  }
  const float2 old0 = xm[0], old1 = xm[1], old2 = xm[2];

  const bool is_qk = hb < 2 * p.n_qk;
  float *dst;
  int dst_stride;
  if (hb < p.n_qk) {
    dst = p.q + hb * kHeadDim;
    dst_stride = p.n_qk * kHeadDim;
  } else if (is_qk) {
    dst = p.k + (hb - p.n_qk) * kHeadDim;
    dst_stride = p.n_qk * kHeadDim;
  } else {
    dst = p.v + (hb - 2 * p.n_qk) * kHeadDim;
    dst_stride = p.n_v * kHeadDim;
  }

  for (int i = 0; i < ntok; ++i) {
    const size_t t = static_cast<size_t>(seq0 + tau0 + i);
    const float2 x = Act<TA>::load2(qkv, t * C + c);
    float y0 = w0.x * xm[0].x + w0.y * xm[1].x + w0.z * xm[2].x + w0.w * x.x;
    float y1 = w1.x * xm[0].y + w1.y * xm[1].y + w1.z * xm[2].y + w1.w * x.y;
    y0 = siluf_(y0);
    y1 = siluf_(y1);
    if (is_qk) {
      const float ss = wave_sum(y0 * y0 + y1 * y1);
      const float inv = 1.0f / fmaxf(sqrtf(ss), p.l2_eps);
      y0 *= inv;
      y1 *= inv;
    }
    *reinterpret_cast<float2 *>(dst + t * dst_stride + 2 * lane) = make_float2(y0, y1);
    xm[0] = xm[1];
    xm[1] = xm[2];
    xm[2] = x;
  }

  if (!is_qk && lane < ntok) {
    const int j = hb - 2 * p.n_qk;
    const size_t e = static_cast<size_t>(seq0 + tau0 + lane) * p.n_v + j;
    const TA *bl = static_cast<const TA *>(p.b);
    const TA *al = static_cast<const TA *>(p.a);
    p.beta[e] = sigmoidf_(Act<TA>::load(bl, e));
    p.g[e] = -expf(p.A_log[j]) * softplusf_(Act<TA>::load(al, e) + p.dt_bias[j]);
  }

  // The first tile of a sequence writes its new conv state: rows L, L+1, L+2
  // of [state; x]. This lane read the old state of exactly these channels
  // above, so an in-place update is safe; no other tile reads the state.
  if (tile == 0) {
#pragma unroll
    for (int r = 0; r < kConvK - 1; ++r) {
      const int src = L + r;
      float2 val;
      if (src >= kConvK - 1) {
        val = Act<TA>::load2(qkv, static_cast<size_t>(seq0 + src - (kConvK - 1)) * C + c);
      } else {
        val = src == 0 ? old0 : (src == 1 ? old1 : old2);
      }
      Act<TA>::store2(st_out, st_base + static_cast<size_t>(r) * C + c, val);
    }
  }
}

}  // namespace

hipError_t launch_prep(const PrepParams &p, gdn_dtype act, hipStream_t s) {
  const int64_t tiles = (static_cast<int64_t>(p.n_tokens) + kPrepTile - 1) / kPrepTile + p.n_seqs;
  const dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(2 * p.n_qk + p.n_v));
  if (act == GDN_BF16)
    hipLaunchKernelGGL(prep_kernel<bf16_t>, grid, dim3(kWave), 0, s, p);
  else
    hipLaunchKernelGGL(prep_kernel<float>, grid, dim3(kWave), 0, s, p);
  return hipGetLastError();
}

}  // namespace gdn
