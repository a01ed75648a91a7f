// decode.hip -- one recurrent delta-rule step for a batch of sequences.
//
// Method: the xwen CLAUDE.md page, section "Architecture cheat sheet", gated
// DeltaNet paragraph, recurrent step (decay, read S.k, delta scaled by beta,
// rank-1 update k outer d, readout of the updated state over sqrt(128)),
// with K/Q-head j mod Hqk for V-head j (tiled repeat).
//
// The step is one streaming pass over the 128x128 fp32 state of each
// (sequence, V-head). Every value column c is independent given k, q, beta
// and g, so a block owns a 128-row x 32-column slab of one head: it reads
// the slab once, forms S.k and S.q for its 32 columns, and writes the slab
// back updated, using
//   u = e^g (S^T k),  d = beta (v - u),  o = (e^g (S^T q) + (k.q) d) / sqrt(128),
//   S' = e^g S + k d^T,
// which equals reading from the decayed and updated state. HBM-bound:
// 2 x 64 KiB of state per (sequence, head) against ~0.75 flop per byte.
//
// Block: 256 threads. Thread t holds rows 4*(t/8) .. +3 and columns
// 4*(t%8) .. +3 of the slab (16 floats): each row segment is a 128-byte
// coalesced access. Column sums are reduced across the 8 row groups of a
// wave with lane shuffles, then across the 4 waves through LDS.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kSlab = 32;
constexpr int kDecodeThreads = 256;

template <typename TA>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeParams p) {
  const int tid = threadIdx.x;
  const int slab = blockIdx.x % (kHeadDim / kSlab);
  const int hv = (blockIdx.x / (kHeadDim / kSlab)) % p.n_v;
  const int n = blockIdx.x / ((kHeadDim / kSlab) * p.n_v);
  const int hk = hv % p.n_qk;
  const int cq = tid & 7;          // column quad
  const int rg = tid >> 3;         // row group (0..31)
  const int row0 = rg * 4;
  const int col0 = slab * kSlab + cq * 4;

  const size_t sbase = (static_cast<size_t>(n) * p.n_v + hv) * kHeadDim * kHeadDim;
  const float *Sin = p.S_in + sbase;
  float4 S[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    S[r] = *reinterpret_cast<const float4 *>(Sin + (row0 + r) * kHeadDim + col0);

  const size_t qk_base = (static_cast<size_t>(n) * p.n_qk + hk) * kHeadDim;
  const float4 kv = *reinterpret_cast<const float4 *>(p.k + qk_base + row0);
  const float4 qv = *reinterpret_cast<const float4 *>(p.q + qk_base + row0);
  const float kr[4] = {kv.x, kv.y, kv.z, kv.w};
  const float qr[4] = {qv.x, qv.y, qv.z, qv.w};

  // Partial column sums over this thread's 4 rows: S^T k, S^T q, and k.q.
  float part[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) part[i] = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    part[0] += S[r].x * kr[r]; part[1] += S[r].y * kr[r];
    part[2] += S[r].z * kr[r]; part[3] += S[r].w * kr[r];
    part[4] += S[r].x * qr[r]; part[5] += S[r].y * qr[r];
    part[6] += S[r].z * qr[r]; part[7] += S[r].w * qr[r];
    part[8] += kr[r] * qr[r];
  }
  // Reduce over the 8 row groups of this wave (lane bits 3..5).
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    float x = part[i];
    x += __shfl_xor(x, 8, kWave);
    x += __shfl_xor(x, 16, kWave);
    x += __shfl_xor(x, 32, kWave);
    part[i] = x;
  }
  __shared__ float red[kDecodeThreads / kWave][8][9];
  const int wave = tid / kWave;
  if ((tid & (kWave - 1)) < 8) {
#pragma unroll
    for (int i = 0; i < 9; ++i) red[wave][cq][i] = part[i];
  }
  __syncthreads();
  float tot[9];
#pragma unroll
  for (int i = 0; i < 9; ++i)
    tot[i] = red[0][cq][i] + red[1][cq][i] + red[2][cq][i] + red[3][cq][i];

  const size_t e = static_cast<size_t>(n) * p.n_v + hv;
  const float eg = expf(p.g[e]);
  const float bt = p.beta[e];
  const float4 vv = *reinterpret_cast<const float4 *>(p.v + e * kHeadDim + col0);
  const float vc[4] = {vv.x, vv.y, vv.z, vv.w};
  const float scale = 0.08838834764831845f;  // 1/sqrt(128)
  float d[4], o[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    d[c] = bt * (vc[c] - eg * tot[c]);
    o[c] = scale * (eg * tot[4 + c] + tot[8] * d[c]);
  }

  float *Sout = p.S_out + sbase;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float4 w;
    w.x = eg * S[r].x + kr[r] * d[0];
    w.y = eg * S[r].y + kr[r] * d[1];
    w.z = eg * S[r].z + kr[r] * d[2];
    w.w = eg * S[r].w + kr[r] * d[3];
    *reinterpret_cast<float4 *>(Sout + (row0 + r) * kHeadDim + col0) = w;
  }
  if (rg == 0) Act<TA>::store4(static_cast<TA *>(p.o), e * kHeadDim + col0, make_float4(o[0], o[1], o[2], o[3]));
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, gdn_dtype act, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(p.n_seqs) * p.n_v * (kHeadDim / kSlab);
  if (act == GDN_BF16)
    hipLaunchKernelGGL(decode_kernel<bf16_t>, dim3(static_cast<unsigned>(blocks)), dim3(kDecodeThreads), 0, s, p);
  else
    hipLaunchKernelGGL(decode_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(kDecodeThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace gdn
