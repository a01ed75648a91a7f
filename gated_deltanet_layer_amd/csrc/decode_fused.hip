// decode_fused.hip -- one decode step of the whole token mixer in one launch:
// conv + SiLU + split + L2 norm + gates for the step's token, the recurrent
// delta-rule update of the 128x128 state, and the gated RMSNorm of the
// readout.
//
// Method: the xwen CLAUDE.md page, section "Architecture cheat sheet", gated
// DeltaNet paragraph: causal depthwise conv (kernel 4, no bias) over the
// fused stream, SiLU over all of it, q | k | v split, x / max(||x||, eps)
// (or the HF form x / sqrt(sum x^2 + eps) the same paragraph notes, by config),
// K-head j mod Hqk for V-head j (tiled repeat), beta = sigmoid(b),
// g = -exp(A_log) softplus(a + dt_bias) (section "GGUF facts that differ
// from the HF checkpoint" for -exp(A_log) and the multiply-ready norm
// weight), then the recurrent step (decay, read S.k, delta, rank-1 update,
// readout of the updated state over sqrt(128)) and the gated RMSNorm
// (norm, times the weight, times silu(z)).
//
// A block owns one (sequence, V-head): it streams the head's 64 KiB state in
// and out once, so the normalisation of the 128 readout values needs no
// other block. The state loads are issued first; while they are in flight,
// waves 0..2 compute q, k (of K-head j mod Hqk) and v of the token, each
// lane two adjacent channels, and one lane the two gates. The state step
// uses
//   u = e^g (S^T k),  d = beta (v - u),  o = (e^g (S^T q) + (k.q) d) / sqrt(128),
//   S' = e^g S + k d^T.
// Thread t holds rows 8 (t / 32) .. +7 and columns 4 (t % 32) .. +3 (32
// floats): each row is read and written as 512 contiguous bytes by 32 lanes.
//
// The new conv state of the V-head's channels is written by its block, that
// of the q and k channels of K-head h by the block of V-head h; other blocks
// read those channels of the old state during the step, so the old and new
// conv states must be different buffers.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kFusedThreads = 512;
constexpr int kFusedWaves = kFusedThreads / kWave;
constexpr int kRowsPerThread = 8;
constexpr int kColQuads = kHeadDim / 4;   // 32 lanes span a row

// Activation inputs in flight travel as their raw bits and are widened to
// fp32 where they are used. Widened at the load, the wave would wait for
// the load right there, and with it (one counter covers loads and stores)
// for every store it issued before, such as the previous token's 64 KiB
// snapshot plane.
template <typename TA> struct Bits;
template <> struct Bits<bf16_t> {
  using X1 = uint32_t;   // one value
  using X2 = uint32_t;   // two adjacent values
  using X4 = uint2;      // four
  static __device__ __forceinline__ X1 get1(const bf16_t *p, size_t i) { return p[i].bits; }
  static __device__ __forceinline__ X2 get2(const bf16_t *p, size_t i) {
    return *reinterpret_cast<const uint32_t *>(p + i);
  }
  static __device__ __forceinline__ X4 get4(const bf16_t *p, size_t i) {
    return *reinterpret_cast<const uint2 *>(p + i);
  }
  static __device__ __forceinline__ void put2(bf16_t *p, size_t i, X2 x) { *reinterpret_cast<uint32_t *>(p + i) = x; }
  static __device__ __forceinline__ float f1(X1 x) { return __uint_as_float(x << 16); }
  static __device__ __forceinline__ float2 f2(X2 w) {
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
  }
  static __device__ __forceinline__ float4 f4(X4 w) {
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
  }
};
template <> struct Bits<float> {
  using X1 = float;
  using X2 = float2;
  using X4 = float4;
  static __device__ __forceinline__ X1 get1(const float *p, size_t i) { return p[i]; }
  static __device__ __forceinline__ X2 get2(const float *p, size_t i) { return *reinterpret_cast<const float2 *>(p + i); }
  static __device__ __forceinline__ X4 get4(const float *p, size_t i) { return *reinterpret_cast<const float4 *>(p + i); }
  static __device__ __forceinline__ void put2(float *p, size_t i, X2 x) { *reinterpret_cast<float2 *>(p + i) = x; }
  static __device__ __forceinline__ float f1(X1 x) { return x; }
  static __device__ __forceinline__ float2 f2(X2 x) { return x; }
  static __device__ __forceinline__ float4 f4(X4 x) { return x; }
};

// kOne: a single token per sequence (gdn_decode_fused), with K = 1 known at
// compile time so that the step keeps the register budget of six waves per
// SIMD.
template <typename TA, bool kOne>
__global__ __launch_bounds__(kFusedThreads) void decode_tokens_kernel(FusedDecodeParams p) {
  __shared__ __attribute__((aligned(16))) float qs[kHeadDim];
  __shared__ __attribute__((aligned(16))) float ks[kHeadDim];
  __shared__ __attribute__((aligned(16))) float vs[kHeadDim];
  __shared__ float gate[2];
  __shared__ float red[kFusedWaves][9][kColQuads];
  __shared__ float tot[9][kColQuads];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();
  const int j = blockIdx.x % p.n_v;
  const int n = blockIdx.x / p.n_v;
  const int hk = j % p.n_qk;
  const int K = kOne ? 1 : p.n_tok;
  const int cq = tid % kColQuads;
  const int row0 = kRowsPerThread * (tid / kColQuads);
  const int col0 = 4 * cq;
  const size_t hd2 = static_cast<size_t>(kHeadDim) * kHeadDim;
  const int C = kHeadDim * (2 * p.n_qk + p.n_v);

  // 1. The state rows of this thread (in flight during the first token's prep).
  float4 S[kRowsPerThread];
  {
    const float *Sin = p.S_in + (static_cast<size_t>(n) * p.n_v + j) * hd2;
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r)
      S[r] = *reinterpret_cast<const float4 *>(Sin + (row0 + r) * kHeadDim + col0);
  }

  // 2. The inputs of token 0, in flight with the state rows: the 4-row conv
  // window, rows -3 .. 0 of [conv state; the sequence's tokens], of two
  // adjacent channels per lane of q (wave 0), k (wave 1) or v (waves 2 and
  // up; only wave 2 uses them), z and the two logits. Every wave loads all of
  // them (same addresses within a wave), so that no load sits in a branch
  // whose end would wait for it. A verify call then issues the next token's
  // loads at the start of each token, the last token reloading its own, and
  // shifts the window by one row at its end.
  using BI = Bits<TA>;
  const int hb = wave == 0 ? hk : (wave == 1 ? p.n_qk + hk : 2 * p.n_qk + j);
  const int ch = hb * kHeadDim + 2 * lane;   // this lane's channel pair
  const TA *xq = static_cast<const TA *>(p.qkv) + static_cast<size_t>(n) * K * C;
  const TA *zp = static_cast<const TA *>(p.z);
  const TA *bp = static_cast<const TA *>(p.b);
  const TA *ap = static_cast<const TA *>(p.a);
  typename BI::X2 xr[kConvK] = {}, xn = {};
  typename BI::X4 zr = {}, zn = {};
  typename BI::X1 br = {}, ar = {}, bn = {}, an = {};
  float4 w0 = make_float4(0.f, 0.f, 0.f, 0.f), w1 = w0, wv = w0;
  const float neg_a = -expf(p.A_log[j]), dtb = p.dt_bias[j];   // the V-head's gate parameters
  if (K > 0) {
    const size_t e0 = static_cast<size_t>(n) * K * p.n_v + j;   // row of z and the logits, token 0
    const TA *st = static_cast<const TA *>(p.st_in) + static_cast<size_t>(n) * (kConvK - 1) * C;
#pragma unroll
    for (int i = 0; i < kConvK - 1; ++i) xr[i] = BI::get2(st, static_cast<size_t>(i) * C + ch);
    xr[kConvK - 1] = BI::get2(xq, ch);
    zr = BI::get4(zp, e0 * kHeadDim + col0);
    br = BI::get1(bp, e0);
    ar = BI::get1(ap, e0);
    w0 = reinterpret_cast<const float4 *>(p.conv_w)[ch];
    w1 = reinterpret_cast<const float4 *>(p.conv_w)[ch + 1];
    wv = *reinterpret_cast<const float4 *>(p.norm_w + col0);
  }

  for (int tau = 0; tau < K; ++tau) {
    const size_t tok = static_cast<size_t>(n) * K + tau;      // row of qkv, z, y, logits
    const size_t e = tok * p.n_v + j;
    const int plane = K - 1 - tau;                             // snapshot plane (most recent first)
    if (tau > 0) __syncthreads();                              // the last token's LDS reads are done
    if constexpr (!kOne) {
      const int tn = min(tau + 1, K - 1);
      const size_t en = (static_cast<size_t>(n) * K + tn) * p.n_v + j;
      xn = BI::get2(xq, static_cast<size_t>(tn) * C + ch);
      zn = BI::get4(zp, en * kHeadDim + col0);
      bn = BI::get1(bp, en);
      an = BI::get1(ap, en);
    }

    // 3. The token's q (wave 0), k (wave 1), v (wave 2); gates (wave 3).
    if (wave < 3) {
      const float2 x0 = BI::f2(xr[0]), x1 = BI::f2(xr[1]), x2 = BI::f2(xr[2]), x3 = BI::f2(xr[3]);
      float y0 = w0.x * x0.x + w0.y * x1.x + w0.z * x2.x + w0.w * x3.x;
      float y1 = w1.x * x0.y + w1.y * x1.y + w1.z * x2.y + w1.w * x3.y;
      y0 = siluf_(y0);
      y1 = siluf_(y1);
      if (wave < 2) {
        const float ss = wave_sum(y0 * y0 + y1 * y1);
        const float inv = l2_inv(ss, p.l2_eps, p.l2_mode == GDN_L2_RSQRT);
        y0 *= inv;
        y1 *= inv;
      }
      float *dst = wave == 0 ? qs : (wave == 1 ? ks : vs);
      *reinterpret_cast<float2 *>(dst + 2 * lane) = make_float2(y0, y1);
      // Conv state after this token: rows tau-2, tau-1, tau, as stored.
      if (wave == 2 || j == hk) {
        TA *so = static_cast<TA *>(p.st_out) + (static_cast<size_t>(n) * K + plane) * (kConvK - 1) * C;
        BI::put2(so, ch, xr[1]);
        BI::put2(so, ch + C, xr[2]);
        BI::put2(so, ch + 2 * C, xr[3]);
      }
    } else if (tid == 3 * kWave) {
      gate[0] = sigmoidf_(BI::f1(br));
      gate[1] = neg_a * softplusf_(BI::f1(ar) + dtb);
    }
    __syncthreads();

    // 4. Column sums S^T k, S^T q over this thread's rows, and k.q.
    float kr[kRowsPerThread], qr[kRowsPerThread];
#pragma unroll
    for (int h = 0; h < kRowsPerThread / 4; ++h) {
      const float4 k4 = *reinterpret_cast<const float4 *>(ks + row0 + 4 * h);
      const float4 q4 = *reinterpret_cast<const float4 *>(qs + row0 + 4 * h);
      kr[4 * h] = k4.x; kr[4 * h + 1] = k4.y; kr[4 * h + 2] = k4.z; kr[4 * h + 3] = k4.w;
      qr[4 * h] = q4.x; qr[4 * h + 1] = q4.y; qr[4 * h + 2] = q4.z; qr[4 * h + 3] = q4.w;
    }
    float part[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) part[i] = 0.0f;
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) {
      part[0] += S[r].x * kr[r]; part[1] += S[r].y * kr[r];
      part[2] += S[r].z * kr[r]; part[3] += S[r].w * kr[r];
      part[4] += S[r].x * qr[r]; part[5] += S[r].y * qr[r];
      part[6] += S[r].z * qr[r]; part[7] += S[r].w * qr[r];
      part[8] += kr[r] * qr[r];
    }
    if constexpr (!kOne) {
      // The state after token tau - 1 is still in S: its snapshot plane goes
      // out here, among this token's reductions, rather than as a burst
      // before the next barrier (the last token's plane follows its update).
      if (tau > 0) {
        float *Sp = p.S_out + ((static_cast<size_t>(n) * K + plane + 1) * p.n_v + j) * hd2;
#pragma unroll
        for (int r = 0; r < kRowsPerThread; ++r) *reinterpret_cast<float4 *>(Sp + (row0 + r) * kHeadDim + col0) = S[r];
      }
    }
    // The two row groups of a wave (lanes l and l + 32 share columns), then
    // the waves through LDS.
#pragma unroll
    for (int i = 0; i < 9; ++i) part[i] += __shfl_xor(part[i], 32, kWave);
    if (lane < kColQuads) {
#pragma unroll
      for (int i = 0; i < 9; ++i) red[wave][i][cq] = part[i];
    }
    __syncthreads();
    if (tid < 9 * kColQuads) {
      const int i = tid / kColQuads, c = tid % kColQuads;
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < kFusedWaves; ++w) s += red[w][i][c];
      tot[i][c] = s;
    }
    __syncthreads();

    // 5. Delta, readout, state update; the updated state is this token's
    // snapshot plane.
    const float bt = gate[0];
    const float eg = expf(gate[1]);
    const float kq = tot[8][cq];
    const float4 v4 = *reinterpret_cast<const float4 *>(vs + col0);
    const float vc[4] = {v4.x, v4.y, v4.z, v4.w};
    const float scale = 0.08838834764831845f;  // 1/sqrt(128)
    float d[4], o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      d[c] = bt * (vc[c] - eg * tot[c][cq]);
      o[c] = scale * (eg * tot[4 + c][cq] + kq * d[c]);
    }
    float *Sout = p.S_out + ((static_cast<size_t>(n) * K + plane) * p.n_v + j) * hd2;
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) {
      S[r].x = eg * S[r].x + kr[r] * d[0];
      S[r].y = eg * S[r].y + kr[r] * d[1];
      S[r].z = eg * S[r].z + kr[r] * d[2];
      S[r].w = eg * S[r].w + kr[r] * d[3];
      if (kOne || tau == K - 1) *reinterpret_cast<float4 *>(Sout + (row0 + r) * kHeadDim + col0) = S[r];
    }

    // 6. Gated RMSNorm of the 128 readout values: each 32-lane half of wave 0
    // holds all of them (4 per lane).
    if (wave == 0) {
      float ss = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
      ss = row16_sum(ss);
      ss += __shfl_xor(ss, 16, kWave);
      const float inv = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + p.norm_eps);
      if (lane < kColQuads) {
        float4 y;
        const float4 zv = BI::f4(zr);
        y.x = o[0] * inv * wv.x * siluf_(zv.x);
        y.y = o[1] * inv * wv.y * siluf_(zv.y);
        y.z = o[2] * inv * wv.z * siluf_(zv.z);
        y.w = o[3] * inv * wv.w * siluf_(zv.w);
        Act<TA>::store4(static_cast<TA *>(p.y), e * kHeadDim + col0, y);
      }
    }

    // The next token's window and inputs.
    if constexpr (!kOne) {
#pragma unroll
      for (int i = 0; i < kConvK - 1; ++i) xr[i] = xr[i + 1];
      xr[kConvK - 1] = xn;
      zr = zn;
      br = bn;
      ar = an;
    }
  }
}

}  // namespace

hipError_t launch_decode_fused(const FusedDecodeParams &p, gdn_dtype act, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(p.n_seqs) * p.n_v;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kFusedThreads);
  if (act == GDN_BF16) {
    if (p.n_tok == 1)
      hipLaunchKernelGGL((decode_tokens_kernel<bf16_t, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((decode_tokens_kernel<bf16_t, false>), grid, block, 0, s, p);
  } else {
    if (p.n_tok == 1)
      hipLaunchKernelGGL((decode_tokens_kernel<float, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((decode_tokens_kernel<float, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace gdn
