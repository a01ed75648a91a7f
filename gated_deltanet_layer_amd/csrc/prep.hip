// prep.hip -- causal depthwise conv (kernel 4, no bias) + SiLU + split +
// clamp-form L2 norm of q/k + beta/g gates, and the conv-state update.
//
// Method: the xwen CLAUDE.md page, section "Architecture cheat sheet", gated
// DeltaNet paragraph (conv over the whole fused width, SiLU over all of it,
// q | k | v split, x / max(||x||, eps) (or the HF form x / sqrt(sum x^2 +
// eps) the same paragraph notes, by config), beta = sigmoid, g = ssm_a * softplus
// with ssm_a = -exp(A_log) per the section "GGUF facts that differ from the
// HF checkpoint").
//
// Grid: x = token tiles (kTile tokens of one sequence; an empty sequence
// owns one tile that only moves its conv state), y = groups of 4 head blocks
// (a head block is 128 fused channels: Hqk q heads, Hqk k heads, Hv v
// heads). One wave per head block, so a block reads 4 adjacent 256-byte
// pieces of every bf16 row; each lane owns 2 adjacent channels and loads the tile's rows plus a 3-row halo
// into registers before computing, so all its loads are in flight together.
// HBM-bound: per token it reads C act values and writes C fp32 values.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kPrepWaves = 4;   // consecutive head blocks per block (1 KB of each bf16 row)

template <typename TA, int kTile>
__global__ __launch_bounds__(kPrepWaves * kWave) void prep_kernel(PrepParams p) {
  const int lane = lane_id();
  const int hb = blockIdx.y * kPrepWaves + threadIdx.x / kWave;
  if (hb >= 2 * p.n_qk + p.n_v) return;
  int n, tile;
  if (!find_unit(p.cu, p.n_seqs, blockIdx.x, kTile, 1, &n, &tile)) return;
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

  const int tau0 = tile * kTile;
  const int ntok = min(kTile, L - tau0);

  // Raw rows tau0 - 3 .. tau0 + kTile - 1 of [state; x], all loaded before
  // any is used.
  // Rows before the sequence come from the conv state; rows past its end are
  // clamped to its last row and never used. An empty sequence reads state
  // rows only, clamped to its 3 rows (those past row 2 are never used).
  constexpr int kRows = kTile + kConvK - 1;
  float2 xr[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int pos = tau0 - (kConvK - 1) + r;
    const bool from_state = pos < 0 || L == 0;
    const TA *src = from_state ? st_in + st_base + static_cast<size_t>(min(max(pos + kConvK - 1, 0), kConvK - 2)) * C
                               : qkv + static_cast<size_t>(seq0 + min(pos, L - 1)) * C;
    xr[r] = Act<TA>::load2(src, c);
  }

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

#pragma unroll
  for (int i = 0; i < kTile; ++i) {
    if (i < ntok) {
      const size_t t = static_cast<size_t>(seq0 + tau0 + i);
      float y0 = w0.x * xr[i].x + w0.y * xr[i + 1].x + w0.z * xr[i + 2].x + w0.w * xr[i + 3].x;
      float y1 = w1.x * xr[i].y + w1.y * xr[i + 1].y + w1.z * xr[i + 2].y + w1.w * xr[i + 3].y;
      y0 = siluf_(y0);
      y1 = siluf_(y1);
      if (is_qk) {
        const float ss = wave_sum(y0 * y0 + y1 * y1);
        const float inv = l2_inv(ss, p.l2_eps, p.l2_mode == GDN_L2_RSQRT);
        y0 *= inv;
        y1 *= inv;
      }
      *reinterpret_cast<float2 *>(dst + t * dst_stride + 2 * lane) = make_float2(y0, y1);
    }
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
  // Written with constant register indices for each short length (rows
  // 0..2 of [state; x] are xr[0..2], token 0 and 1 are xr[3] and xr[4]).
  if (tile == 0) {
    float2 s0, s1, s2;
    if (L == 0) {
      s0 = xr[0]; s1 = xr[1]; s2 = xr[2];
    } else if (L == 1) {
      s0 = xr[1]; s1 = xr[2]; s2 = xr[3];
    } else if (L == 2) {
      s0 = xr[2]; s1 = xr[3]; s2 = xr[4];
    } else {
      const size_t r0 = static_cast<size_t>(seq0 + L - (kConvK - 1)) * C + c;
      s0 = Act<TA>::load2(qkv, r0);
      s1 = Act<TA>::load2(qkv, r0 + C);
      s2 = Act<TA>::load2(qkv, r0 + 2 * static_cast<size_t>(C));
    }
    Act<TA>::store2(st_out, st_base + c, s0);
    Act<TA>::store2(st_out, st_base + C + c, s1);
    Act<TA>::store2(st_out, st_base + 2 * static_cast<size_t>(C) + c, s2);
  }
}

}  // namespace

hipError_t launch_prep(const PrepParams &p, gdn_dtype act, hipStream_t s) {
  const int tile = prep_tile(p.n_seqs, p.n_tokens);
  const int64_t tiles = (static_cast<int64_t>(p.n_tokens) + tile - 1) / tile + p.n_seqs;
  const int head_blocks = 2 * p.n_qk + p.n_v;
  const dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>((head_blocks + kPrepWaves - 1) / kPrepWaves));
  const dim3 block(kPrepWaves * kWave);
  if (act == GDN_BF16) {
    if (tile == 32) hipLaunchKernelGGL((prep_kernel<bf16_t, 32>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((prep_kernel<bf16_t, 8>), grid, block, 0, s, p);
  } else {
    if (tile == 32) hipLaunchKernelGGL((prep_kernel<float, 32>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((prep_kernel<float, 8>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace gdn
