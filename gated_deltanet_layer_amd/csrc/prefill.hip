// prefill.hip -- the delta rule in its chunked form (chunks of 64 tokens).
//
// Method: the recurrent step of the xwen CLAUDE.md page (section
// "Architecture cheat sheet", gated DeltaNet paragraph), rewritten exactly
// over chunks of 64 tokens (the chunk length the page's section "Ground
// truth, in order of authority" names). Within a chunk of n tokens, with
// start state S0, log-decays g, cumulative sums gam and Gam = exp(gam):
//   A[r][m] = beta_r exp(gam_r - gam_m) k_r.k_m     (m < r)
//   P[r][m] = exp(gam_r - gam_m) q_r.k_m            (m <= r)
//   Tm      = (I + A)^-1 diag(beta)
//   D       = Tm (V - diag(Gam) K S0)                (row r = the delta of token r)
//   O       = s (diag(Gam) Q S0 + P D)               (s = 1/sqrt(128))
//   S_end   = Gam_n S0 + (diag(exp(gam_n - gam)) K)^T D
// Unrolling the recurrent step from S0 gives these identities; only the
// last three lines depend on S0.
//
// Two kernels:
//  * chunk_local: one block per (chunk, K-head). Builds K K^T and Q K^T once
//    for the K-head, then for each V-head that uses it (tiled repeat: V-heads
//    h, h + Hqk, ...) applies that head's decays and beta, writes P, and
//    inverts the unit lower-triangular I + A by blocked forward substitution
//    on 16x16 blocks (diagonal blocks by substitution, off-diagonal blocks by
//    fp32 MFMA products), writing Tm and gam to the workspace.
//  * chunk_state: one block per (sequence, V-head, 32-column slab of S). The
//    value columns of S are independent, so four blocks share a head. It
//    walks the sequence's chunks in order with the fp32 state slab held in
//    MFMA accumulators: [K; Q] S, D = Tm (V - Gam K S), O = s(Gam Q S + P D),
//    S <- Gam_n S + K~^T D.
// Every product runs at fp32-grade precision: fp32 MFMA for fp32
// activations, three-pass split bf16 MFMA (hi*hi + hi*lo + lo*hi) for bf16
// activations. The gated RMSNorm downstream divides by sqrt(mean(o^2) + 1e-6),
// which magnifies absolute errors of low-energy rows of o by up to 1e3, so a
// single bf16 pass is not accurate enough.
//
// Decays: exp is only taken of gam_r - gam_m with m <= r (never positive),
// so nothing overflows; exp(gam) may underflow to 0, which is harmless.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kSlab = 32;                 // state columns per chunk_state block
constexpr int kLdK = kHeadDim + 4;        // LDS row pitch of K/Q/S^T (floats)
constexpr int kLdC = kChunk + 4;          // LDS row pitch of 64-wide matrices
constexpr int kChunkMat = kChunk * kChunk;

struct Workspace {
  float *T;    // [max_chunks][Hv][64][64]
  float *P;    // [max_chunks][Hv][64][64]
  double *gam; // [max_chunks][Hv][64] cumulative log-decay inside the chunk
};

__host__ __device__ inline Workspace carve(void *ws, int64_t max_chunks, int n_v) {
  Workspace w;
  float *base = static_cast<float *>(ws);
  const int64_t mats = max_chunks * n_v * kChunkMat;
  w.T = base;
  w.P = base + mats;
  w.gam = reinterpret_cast<double *>(base + 2 * mats);
  return w;
}

// Load rows [t0, t0+len) of one head (128 fp32 per row, row stride `stride`)
// into LDS rows 0..63 (zero past len).
__device__ __forceinline__ void load_rows(float *dst, const float *src, int stride, int len) {
  for (int idx = threadIdx.x; idx < kChunk * (kHeadDim / 4); idx += kThreads) {
    const int r = idx / (kHeadDim / 4);
    const int c4 = idx % (kHeadDim / 4);
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < len) x = *reinterpret_cast<const float4 *>(src + static_cast<size_t>(r) * stride + 4 * c4);
    *reinterpret_cast<float4 *>(dst + r * kLdK + 4 * c4) = x;
  }
}

template <Prec P>
__global__ __launch_bounds__(kThreads) void chunk_local_kernel(PrefillParams p, int64_t max_chunks) {
  __shared__ float Ks[kChunk * kLdK];
  __shared__ float Qs[kChunk * kLdK];
  __shared__ float Gkk[kChunk * kLdC];
  __shared__ float Gqk[kChunk * kLdC];
  __shared__ float Lm[kChunk * kLdC];
  __shared__ float Xm[kChunk * kLdC];
  __shared__ float Tsc[4][16 * 17];
  __shared__ double gam_s[kChunk];
  __shared__ float bet_s[kChunk];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();
  const int h = blockIdx.y;
  int n, ci;
  if (!find_unit(p.cu, p.n_seqs, blockIdx.x, kChunk, 0, &n, &ci)) return;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  if (seq0 < 0 || L < 0 || seq0 + L > p.n_tokens) return;
  const int t0 = seq0 + ci * kChunk;
  const int len = min(kChunk, L - ci * kChunk);
  const int cid = blockIdx.x;
  const Workspace ws = carve(p.ws, max_chunks, p.n_v);

  const int qk_stride = p.n_qk * kHeadDim;
  load_rows(Ks, p.k + static_cast<size_t>(t0) * qk_stride + h * kHeadDim, qk_stride, len);
  load_rows(Qs, p.q + static_cast<size_t>(t0) * qk_stride + h * kHeadDim, qk_stride, len);
  __syncthreads();

  // Lower-triangular 16x16 tiles of K K^T and Q K^T (10 each).
  for (int tile = wave; tile < 32; tile += 4) {
    const int which = tile / 16, rt = (tile % 16) / 4, ct = tile % 4;
    if (ct > rt) continue;
    const float *A = which ? Qs : Ks;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 32; ++ks)
      Mma<P>::run(acc, frag_rows(A, kLdK, rt * 16, ks * 32), frag_rows(Ks, kLdK, ct * 16, ks * 32));
    float *G = which ? Gqk : Gkk;
#pragma unroll
    for (int r = 0; r < 4; ++r) G[(rt * 16 + acc_row(r)) * kLdC + ct * 16 + acc_col()] = acc[r];
  }
  __syncthreads();

  for (int j = h; j < p.n_v; j += p.n_qk) {
    // Cumulative log-decay (0 past len, so gam stays at its last value) and
    // beta. gam reaches a few hundred inside a chunk and only its differences
    // gam_r - gam_m are used: in fp32 they would lose ~|gam| * 6e-8 to
    // cancellation, so the scan and the differences are fp64.
    if (wave == 0) {
      const size_t e = static_cast<size_t>(t0 + lane) * p.n_v + j;
      const double gr = lane < len ? static_cast<double>(p.g[e]) : 0.0;
      const float br = lane < len ? p.beta[e] : 0.f;
      const double gm = wave_inclusive_scan_d(gr);
      gam_s[lane] = gm;
      bet_s[lane] = br;
      ws.gam[(static_cast<size_t>(cid) * p.n_v + j) * kChunk + lane] = gm;
    }
    __syncthreads();

    float *Pout = ws.P + (static_cast<size_t>(cid) * p.n_v + j) * kChunkMat;
    for (int idx = tid; idx < kChunkMat; idx += kThreads) {
      const int r = idx / kChunk, m = idx % kChunk;
      float lv = r == m ? 1.f : 0.f, pv = 0.f;
      if (m <= r) {
        const float dec = expf(static_cast<float>(gam_s[r] - gam_s[m]));
        pv = dec * Gqk[r * kLdC + m];
        if (m < r) lv = bet_s[r] * dec * Gkk[r * kLdC + m];
      }
      Lm[r * kLdC + m] = lv;
      Xm[r * kLdC + m] = 0.f;
      Pout[idx] = pv;
    }
    __syncthreads();

    // Diagonal blocks: X_bb = L_bb^-1 by forward substitution, one column per lane.
    if (lane < 16) {
      const int b = wave, c = lane;
      const float *Lb = Lm + (b * 16) * kLdC + b * 16;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = r == c ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) acc -= Lb[r * kLdC + m] * x[m];
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Xm[(b * 16 + r) * kLdC + b * 16 + c] = x[r];
    }
    __syncthreads();

    // Off-diagonal blocks, block row by block row:
    //   X_ij = -X_ii * sum_{k=j}^{i-1} L_ik X_kj   (wave j computes X_ij)
    for (int bi = 1; bi < 4; ++bi) {
      const int bj = wave;
      if (bj < bi) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int bk = bj; bk < bi; ++bk) {
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) {
            const float a = Lm[(bi * 16 + (lane & 15)) * kLdC + bk * 16 + 4 * k4 + (lane >> 4)];
            const float b = Xm[(bk * 16 + 4 * k4 + (lane >> 4)) * kLdC + bj * 16 + (lane & 15)];
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Tsc[wave][acc_row(r) * 17 + acc_col()] = acc[r];
      }
      __syncthreads();
      if (bj < bi) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const float a = Xm[(bi * 16 + (lane & 15)) * kLdC + bi * 16 + 4 * k4 + (lane >> 4)];
          const float b = Tsc[wave][(4 * k4 + (lane >> 4)) * 17 + (lane & 15)];
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Xm[(bi * 16 + acc_row(r)) * kLdC + bj * 16 + acc_col()] = -acc[r];
      }
      __syncthreads();
    }

    // Tm = X diag(beta).
    float *Tout = ws.T + (static_cast<size_t>(cid) * p.n_v + j) * kChunkMat;
    for (int idx = tid; idx < kChunkMat; idx += kThreads) {
      const int r = idx / kChunk, m = idx % kChunk;
      Tout[idx] = m <= r ? Xm[r * kLdC + m] * bet_s[m] : 0.f;
    }
    __syncthreads();
  }
}

template <Prec P, typename TA>
__global__ __launch_bounds__(kThreads) void chunk_state_kernel(PrefillParams p, int64_t max_chunks) {
  __shared__ float Ks[kChunk * kLdK];
  __shared__ float Qs[kChunk * kLdK];
  __shared__ float St[kSlab * kLdK];       // S^T of the slab: St[c][i]
  __shared__ float Tms[kChunk * kLdC];
  __shared__ float Ps[kChunk * kLdC];
  __shared__ float Rt[kSlab * kLdC];       // R^T: Rt[c][r]
  __shared__ float Dt[kSlab * kLdC];       // D^T: Dt[c][r]
  __shared__ float G_s[kChunk];            // exp(gam_r)
  __shared__ float ksc_s[kChunk];          // exp(gam_end - gam_r)

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();
  const int nslab = kHeadDim / kSlab;
  const int slab = blockIdx.x % nslab;
  const int j = (blockIdx.x / nslab) % p.n_v;
  const int n = blockIdx.x / (nslab * p.n_v);
  const int hk = j % p.n_qk;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  if (seq0 < 0 || L < 0 || seq0 + L > p.n_tokens) return;
  const int nchunks = (L + kChunk - 1) / kChunk;
  const int cid0 = first_unit(p.cu, n, kChunk, 0);
  // Chunk ids past the workspace only arise from cu_seqlens outside the
  // contract; never index past the workspace.
  if (cid0 + nchunks > max_chunks) return;
  const Workspace ws = carve(p.ws, max_chunks, p.n_v);
  const float scale = 0.08838834764831845f;  // 1/sqrt(128)
  const int col_base = slab * kSlab;

  // State slab in accumulators: wave w owns rows i in [32w, 32w+32), two
  // 16-row tiles x two 16-column tiles; element r of lane l is
  // S[32w + 16 rt + 4(l/16) + r][16 ct + l%16].
  const size_t sbase = (static_cast<size_t>(n) * p.n_v + j) * kHeadDim * kHeadDim;
  f32x4 S[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 32 * wave + 16 * rt + acc_row(r);
        S[rt][ct][r] = p.S_in[sbase + static_cast<size_t>(i) * kHeadDim + col_base + 16 * ct + acc_col()];
      }
  auto write_st = [&]() {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int i = 32 * wave + 16 * rt + acc_row(0);
        *reinterpret_cast<float4 *>(St + (16 * ct + acc_col()) * kLdK + i) =
            make_float4(S[rt][ct][0], S[rt][ct][1], S[rt][ct][2], S[rt][ct][3]);
      }
  };
  write_st();

  const int qk_stride = p.n_qk * kHeadDim;
  const int v_stride = p.n_v * kHeadDim;
  TA *o = static_cast<TA *>(p.o);

  for (int ci = 0; ci < nchunks; ++ci) {
    const int t0 = seq0 + ci * kChunk;
    const int len = min(kChunk, L - ci * kChunk);
    const size_t wsi = static_cast<size_t>(cid0 + ci) * p.n_v + j;
    __syncthreads();
    load_rows(Ks, p.k + static_cast<size_t>(t0) * qk_stride + hk * kHeadDim, qk_stride, len);
    load_rows(Qs, p.q + static_cast<size_t>(t0) * qk_stride + hk * kHeadDim, qk_stride, len);
    for (int idx = tid; idx < kChunkMat / 4; idx += kThreads) {
      const int r = idx / (kChunk / 4), c4 = idx % (kChunk / 4);
      *reinterpret_cast<float4 *>(Tms + r * kLdC + 4 * c4) =
          *reinterpret_cast<const float4 *>(ws.T + wsi * kChunkMat + r * kChunk + 4 * c4);
      *reinterpret_cast<float4 *>(Ps + r * kLdC + 4 * c4) =
          *reinterpret_cast<const float4 *>(ws.P + wsi * kChunkMat + r * kChunk + 4 * c4);
    }
    if (tid < kChunk) {
      const double *gm = ws.gam + wsi * kChunk;
      const double gr = gm[tid];
      G_s[tid] = expf(static_cast<float>(gr));
      ksc_s[tid] = expf(static_cast<float>(gm[kChunk - 1] - gr));
    }
    __syncthreads();
    const float g_end = G_s[kChunk - 1];

    // X = K S (rows 16w..) and Y = Q S (rows 16w..), 16x32 each.
    f32x4 X[2], Y[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      X[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      Y[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kHeadDim / 32; ++ks) {
        const Frag b = frag_rows(St, kLdK, 16 * ct, 32 * ks);
        Mma<P>::run(X[ct], frag_rows(Ks, kLdK, 16 * wave, 32 * ks), b);
        Mma<P>::run(Y[ct], frag_rows(Qs, kLdK, 16 * wave, 32 * ks), b);
      }
    }
    // R = V - diag(Gam) X, stored transposed.
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float rv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * wave + acc_row(r);
        const float vv = row < len ? p.v[static_cast<size_t>(t0 + row) * v_stride + j * kHeadDim + col_base +
                                          16 * ct + acc_col()]
                                   : 0.f;
        rv[r] = vv - G_s[row] * X[ct][r];
      }
      *reinterpret_cast<float4 *>(Rt + (16 * ct + acc_col()) * kLdC + 16 * wave + acc_row(0)) =
          make_float4(rv[0], rv[1], rv[2], rv[3]);
    }
    __syncthreads();

    // D = Tm R (rows 16w..).
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kChunk / 32; ++ks)
        Mma<P>::run(acc, frag_rows(Tms, kLdC, 16 * wave, 32 * ks), frag_rows(Rt, kLdC, 16 * ct, 32 * ks));
      *reinterpret_cast<float4 *>(Dt + (16 * ct + acc_col()) * kLdC + 16 * wave + acc_row(0)) =
          make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();

    // O = s (diag(Gam) Y + P D), rows 16w..
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kChunk / 32; ++ks)
        Mma<P>::run(acc, frag_rows(Ps, kLdC, 16 * wave, 32 * ks), frag_rows(Dt, kLdC, 16 * ct, 32 * ks));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * wave + acc_row(r);
        if (row < len)
          Act<TA>::store(o, static_cast<size_t>(t0 + row) * v_stride + j * kHeadDim + col_base + 16 * ct + acc_col(),
                         scale * (G_s[row] * Y[ct][r] + acc[r]));
      }
    }

    // S <- Gam_n S + K~^T D, with K~[r] = exp(gam_n - gam_r) K[r].
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f32x4 acc = S[rt][ct] * g_end;
#pragma unroll
        for (int ks = 0; ks < kChunk / 32; ++ks)
          Mma<P>::run(acc, frag_cols_scaled(Ks, kLdK, 32 * wave + 16 * rt, 32 * ks, ksc_s),
                      frag_rows(Dt, kLdC, 16 * ct, 32 * ks));
        S[rt][ct] = acc;
      }
    write_st();   // St is not read again until after the next chunk's barrier
  }

#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 32 * wave + 16 * rt + acc_row(r);
        p.S_out[sbase + static_cast<size_t>(i) * kHeadDim + col_base + 16 * ct + acc_col()] = S[rt][ct][r];
      }
}

}  // namespace

size_t prefill_workspace_bytes(int n_seqs, int n_tokens, int n_v) {
  const int64_t chunks = max_chunks(n_seqs, n_tokens);
  return static_cast<size_t>(chunks) * n_v * (2 * kChunkMat * sizeof(float) + kChunk * sizeof(double));
}

hipError_t launch_prefill(const PrefillParams &p, gdn_dtype act, hipStream_t s) {
  const int64_t chunks = max_chunks(p.n_seqs, p.n_tokens);
  const dim3 grid_local(static_cast<unsigned>(chunks), static_cast<unsigned>(p.n_qk));
  const dim3 grid_state(static_cast<unsigned>(static_cast<int64_t>(p.n_seqs) * p.n_v * (kHeadDim / kSlab)));
  if (act == GDN_BF16) {
    if (p.n_tokens > 0) hipLaunchKernelGGL(chunk_local_kernel<Prec::BF16X3>, grid_local, dim3(kThreads), 0, s, p, chunks);
    hipLaunchKernelGGL((chunk_state_kernel<Prec::BF16X3, bf16_t>), grid_state, dim3(kThreads), 0, s, p, chunks);
  } else {
    if (p.n_tokens > 0) hipLaunchKernelGGL(chunk_local_kernel<Prec::F32>, grid_local, dim3(kThreads), 0, s, p, chunks);
    hipLaunchKernelGGL((chunk_state_kernel<Prec::F32, float>), grid_state, dim3(kThreads), 0, s, p, chunks);
  }
  return hipGetLastError();
}

}  // namespace gdn
