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
// activations. Operands are split once, when they are written to LDS (or to
// the workspace), never per use. The gated RMSNorm downstream divides by sqrt(mean(o^2) + 1e-6),
// which magnifies absolute errors of low-energy rows of o by up to 1e3, so a
// single bf16 pass is not accurate enough.
//
// Decays: exp is only taken of gam_r - gam_m with m <= r (never positive),
// so nothing overflows; exp(gam) may underflow to 0, which is harmless.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kLocalThreads = 256;        // chunk_local: 4 waves
constexpr int kStateThreads = 512;        // chunk_state: 8 waves
constexpr int kSlab = 32;                 // state columns per chunk_state block
constexpr int kChunkMat = kChunk * kChunk;
// Row pitches (bytes) of blocked operands in LDS: 128 or 64 contraction
// indices (16 or 8 blocks of 32 bytes) plus 16 bytes to spread LDS banks.
constexpr int kPitch128 = (kHeadDim / 8) * kBlk + 16;   // 528
constexpr int kPitch64 = (kChunk / 8) * kBlk + 16;      // 272
constexpr int kWsPitch = (kChunk / 8) * kBlk;           // 256: workspace rows, unpadded
constexpr int kLdS = kChunk + 1;          // fp32 pitch of the solve's scalar matrices
constexpr int kLdV = kSlab + 4;           // fp32 pitch of the V slab in LDS
constexpr int kLdO = kSlab;               // fp32 pitch of the O staging rows (4 waves x 16 rows fit the R^T buffer)

struct Workspace {
  uint8_t *T;  // [max_chunks][Hv][64 rows][256 B]  Tm, blocked operand rows
  uint8_t *P;  // [max_chunks][Hv][64 rows][256 B]  P, blocked operand rows
  double *gam; // [max_chunks][Hv][64] cumulative log-decay inside the chunk
};

__host__ __device__ inline Workspace carve(void *ws, int64_t max_chunks, int n_v) {
  Workspace w;
  uint8_t *base = static_cast<uint8_t *>(ws);
  const int64_t mat_bytes = max_chunks * n_v * kChunk * kWsPitch;
  w.T = base;
  w.P = base + mat_bytes;
  w.gam = reinterpret_cast<double *>(base + 2 * mat_bytes);
  return w;
}

// An operand fragment from 8 fp32 values (split on the fly).
template <Prec P> __device__ __forceinline__ typename Op<P>::Frag make_frag(f32x4 a, f32x4 b);
template <> __device__ __forceinline__ Op<Prec::F32>::Frag make_frag<Prec::F32>(f32x4 a, f32x4 b) {
  Op<Prec::F32>::Frag f;
  f.a = a;
  f.b = b;
  return f;
}
template <> __device__ __forceinline__ Op<Prec::BF16X3>::Frag make_frag<Prec::BF16X3>(f32x4 a, f32x4 b) {
  Op<Prec::BF16X3>::Frag f;
  bf16x4 ha, la, hb, lb;
  split4(a, ha, la);
  split4(b, hb, lb);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.hi[e] = ha[e]; f.hi[e + 4] = hb[e];
    f.lo[e] = la[e]; f.lo[e + 4] = lb[e];
  }
  return f;
}

// ---------------------------------------------------------------------------
// chunk_local: per (chunk, K-head). ~72 KB of LDS, two blocks per CU.
template <Prec P>
__global__ __launch_bounds__(kLocalThreads) void chunk_local_kernel(PrefillParams p, int64_t max_chunks) {
  // Phase 1 holds K as blocked operand rows; phase 2 reuses the bytes for
  // the fp32 matrices L = I + A and X = L^-1 of the solve.
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[kChunk * kPitch128];
  __shared__ float Gkk[kChunk * kLdS];
  __shared__ float Gqk[kChunk * kLdS];
  __shared__ float Tsc[4][16 * 17];
  __shared__ double gam_s[kChunk];
  __shared__ float bet_s[kChunk];
  uint8_t *Kb = kbuf;
  float *Lm = reinterpret_cast<float *>(kbuf);
  float *Xm = Lm + kChunk * kLdS;

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
  const size_t qk_stride = static_cast<size_t>(p.n_qk) * kHeadDim;
  const float *kg = p.k + t0 * qk_stride + h * kHeadDim;
  const float *qg = p.q + t0 * qk_stride + h * kHeadDim;

  {  // K rows -> blocked operand rows in LDS (rows >= len are zero).
    constexpr int kPer = kChunk * (kHeadDim / 4) / kLocalThreads;
    f32x4 buf[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = tid + u * kLocalThreads, r = idx / (kHeadDim / 4), c4 = idx % (kHeadDim / 4);
      const f32x4 x = *reinterpret_cast<const f32x4 *>(kg + min(r, len - 1) * qk_stride + 4 * c4);
      buf[u] = r < len ? x : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = tid + u * kLocalThreads, r = idx / (kHeadDim / 4), c4 = idx % (kHeadDim / 4);
      Op<P>::put4(Kb + r * kPitch128, 4 * c4, buf[u]);
    }
  }
  block_sync_lds();

  // The 10 lower-triangular 16x16 tiles of K K^T and of Q K^T (Q straight from global).
  for (int tile = wave; tile < 20; tile += 4) {
    const int which = tile / 10, tt = tile % 10;
    int rt = 0;
    while ((rt + 1) * (rt + 2) / 2 <= tt) ++rt;
    const int ct = tt - rt * (rt + 1) / 2;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int qrow = rt * 16 + (lane & 15);
    const float *qp = qg + min(qrow, len - 1) * qk_stride + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 32; ++ks) {
      typename Op<P>::Frag a;
      if (which) {
        f32x4 x0 = *reinterpret_cast<const f32x4 *>(qp + ks * 32);
        f32x4 x1 = *reinterpret_cast<const f32x4 *>(qp + ks * 32 + 4);
        if (qrow >= len) x0 = x1 = f32x4{0.f, 0.f, 0.f, 0.f};
        a = make_frag<P>(x0, x1);
      } else {
        a = frag<P>(Kb, kPitch128, rt * 16, ks * 32);
      }
      Op<P>::mma(acc, a, frag<P>(Kb, kPitch128, ct * 16, ks * 32));
    }
    float *G = which ? Gqk : Gkk;
#pragma unroll
    for (int r = 0; r < 4; ++r) G[(rt * 16 + acc_row(r)) * kLdS + ct * 16 + acc_col()] = acc[r];
  }
  block_sync_lds();   // K is dead from here: kbuf becomes L and X

  for (int j = h; j < p.n_v; j += p.n_qk) {
    // Cumulative log-decay (0 past len, so gam stays at its last value) and
    // beta. gam reaches a few hundred inside a chunk and only its differences
    // gam_r - gam_m are used: in fp32 they would lose ~|gam| * 6e-8 to
    // cancellation, so the scan and the differences are fp64.
    if (wave == 0) {
      const size_t e = static_cast<size_t>(t0 + min(lane, len - 1)) * p.n_v + j;
      const double gr = lane < len ? static_cast<double>(p.g[e]) : 0.0;
      const float br = lane < len ? p.beta[e] : 0.f;
      const double gm = wave_inclusive_scan_d(gr);
      gam_s[lane] = gm;
      bet_s[lane] = br;
      ws.gam[(static_cast<size_t>(cid) * p.n_v + j) * kChunk + lane] = gm;
    }
    block_sync_lds();

    const size_t wsm = (static_cast<size_t>(cid) * p.n_v + j) * kChunk * kWsPitch;
    // L = I + A into LDS and P to the workspace, 4 consecutive m per item.
    for (int it = tid; it < kChunkMat / 4; it += kLocalThreads) {
      const int r = it / (kChunk / 4), m0 = 4 * (it % (kChunk / 4));
      f32x4 pv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + e;
        float lv = r == m ? 1.f : 0.f;
        if (m <= r) {
          const float dec = expf(static_cast<float>(gam_s[r] - gam_s[m]));
          pv[e] = dec * Gqk[r * kLdS + m];
          if (m < r) lv = bet_s[r] * dec * Gkk[r * kLdS + m];
        }
        Lm[r * kLdS + m] = lv;
        Xm[r * kLdS + m] = 0.f;
      }
      Op<P>::put4(ws.P + wsm + r * kWsPitch, m0, pv);
    }
    block_sync_lds();

    // Diagonal blocks: X_bb = L_bb^-1 by forward substitution, one column per lane.
    if (lane < 16) {
      const int b = wave, c = lane;
      const float *Lb = Lm + (b * 16) * kLdS + b * 16;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = r == c ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) acc -= Lb[r * kLdS + m] * x[m];
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Xm[(b * 16 + r) * kLdS + b * 16 + c] = x[r];
    }
    block_sync_lds();

    // Off-diagonal blocks, block row by block row:
    //   X_ij = -X_ii * sum_{k=j}^{i-1} L_ik X_kj   (wave j computes X_ij)
    for (int bi = 1; bi < 4; ++bi) {
      const int bj = wave;
      if (bj < bi) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int bk = bj; bk < bi; ++bk) {
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) {
            const float a = Lm[(bi * 16 + (lane & 15)) * kLdS + bk * 16 + 4 * k4 + (lane >> 4)];
            const float b = Xm[(bk * 16 + 4 * k4 + (lane >> 4)) * kLdS + bj * 16 + (lane & 15)];
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Tsc[wave][acc_row(r) * 17 + acc_col()] = acc[r];
      }
      block_sync_lds();
      if (bj < bi) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const float a = Xm[(bi * 16 + (lane & 15)) * kLdS + bi * 16 + 4 * k4 + (lane >> 4)];
          const float b = Tsc[wave][(4 * k4 + (lane >> 4)) * 17 + (lane & 15)];
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Xm[(bi * 16 + acc_row(r)) * kLdS + bj * 16 + acc_col()] = -acc[r];
      }
      block_sync_lds();
    }

    // Tm = X diag(beta) to the workspace.
    for (int it = tid; it < kChunkMat / 4; it += kLocalThreads) {
      const int r = it / (kChunk / 4), m0 = 4 * (it % (kChunk / 4));
      f32x4 tv;
#pragma unroll
      for (int e = 0; e < 4; ++e) tv[e] = m0 + e <= r ? Xm[r * kLdS + m0 + e] * bet_s[m0 + e] : 0.f;
      Op<P>::put4(ws.T + wsm + r * kWsPitch, m0, tv);
    }
    block_sync_lds();
  }
}

// ---------------------------------------------------------------------------
// chunk_state: per (sequence, V-head, 32-column slab). 8 waves. While chunk
// c is computed, chunk c+1's K, Q, Tm, P, V and gam are loaded into
// registers; they are written to LDS after chunk c's last LDS read.
//
// Work per chunk (wave w, rt = w % 4):
//   X/Y : waves 0-3 X = K S, waves 4-7 Y = Q S, rows 16 rt, both column tiles
//   R   : waves 0-3 R = V - diag(Gam) X  -> R^T in LDS
//   D   : wave w tile (rt, w / 4) of Tm R  -> D^T and (diag(k~) D)^T in LDS,
//         k~_r = exp(gam_n - gam_r)
//   O   : waves 4-7 O = s (diag(Gam) Y + P D), rows 16 rt
//   S   : wave w state rows 16 w: S <- Gam_n S + K^T diag(k~) D
template <Prec P, typename TA>
__global__ __launch_bounds__(kStateThreads) void chunk_state_kernel(PrefillParams p, int64_t max_chunks) {
  __shared__ __attribute__((aligned(16))) uint8_t Kb[kChunk * kPitch128];    // K rows, blocked over i
  __shared__ __attribute__((aligned(16))) uint8_t Qb[kChunk * kPitch128];    // Q rows
  __shared__ __attribute__((aligned(16))) uint8_t Stb[kSlab * kPitch128];    // S^T rows c, blocked over i
  __shared__ __attribute__((aligned(16))) uint8_t Tb[kChunk * kPitch64];     // Tm rows r, blocked over m
  __shared__ __attribute__((aligned(16))) uint8_t Pb[kChunk * kPitch64];     // P rows r
  __shared__ __attribute__((aligned(16))) uint8_t Rtb[kSlab * kPitch64];     // R^T rows c, blocked over r
  __shared__ __attribute__((aligned(16))) uint8_t Dtb[kSlab * kPitch64];     // D^T
  __shared__ __attribute__((aligned(16))) uint8_t Dsb[kSlab * kPitch64];     // (diag(k~) D)^T
  __shared__ float G_s[kChunk];            // exp(gam_r)
  __shared__ float ksc_s[kChunk];          // exp(gam_n - gam_r)
  __shared__ __attribute__((aligned(16))) float Vs[kChunk * kLdV];   // V rows of the slab (fp32)

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();
  const int rt = wave & 3;
  const bool x_wave = wave < 4;
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
  const size_t qk_stride = static_cast<size_t>(p.n_qk) * kHeadDim;
  const size_t v_stride = static_cast<size_t>(p.n_v) * kHeadDim;
  TA *o = static_cast<TA *>(p.o);

  // State rows [16 wave, 16 wave + 16) x the slab's 32 columns, in accumulators:
  // element r of lane l of S[ct] is S[16 wave + 4(l/16) + r][16 ct + l%16].
  const size_t sbase = (static_cast<size_t>(n) * p.n_v + j) * kHeadDim * kHeadDim;
  f32x4 S[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[ct][r] = p.S_in[sbase + static_cast<size_t>(16 * wave + acc_row(r)) * kHeadDim + col_base + 16 * ct + acc_col()];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) put_acc_t<P>(Stb, kPitch128, 16 * wave, 16 * ct, S[ct]);

  // Prefetch registers for one chunk.
  constexpr int kRowsPer = kChunk * (kHeadDim / 4) / kStateThreads;    // f32x4 of K (and of Q) per thread
  constexpr int kMatPer = kChunk * kWsPitch / 16 / kStateThreads;      // 16-byte pieces of Tm (and of P)
  f32x4 pk[kRowsPer], pq[kRowsPer];
  static_assert(kMatPer == 2, "two 16-byte pieces of Tm and of P per thread");
  uint4 pt0, pt1, pp0, pp1;
  f32x4 pvv = {0.f, 0.f, 0.f, 0.f};   // one 16-byte piece of the V slab
  // Per-thread pieces: K/Q rows r_u = (tid + u * 512) / 32, 4 floats at 4 * (tid % 32);
  // V row tid / 8, 4 floats at 4 * (tid % 8).
  const int kq_c4 = tid % (kHeadDim / 4);
  const int v_row = tid / (kSlab / 4), v_c4 = tid % (kSlab / 4);
  double pg = 0.0, pg_end = 0.0;

#define GDN_PREFETCH(c)                                                                              \
  do {                                                                                               \
    const int t0_ = seq0 + (c) * kChunk;                                                             \
    const int len_ = min(kChunk, L - (c) * kChunk);                                                  \
    const float *kg = p.k + t0_ * qk_stride + hk * kHeadDim + 4 * kq_c4;                             \
    const float *qg = p.q + t0_ * qk_stride + hk * kHeadDim + 4 * kq_c4;                             \
    _Pragma("unroll") for (int u = 0; u < kRowsPer; ++u) {                                           \
      const int r = (tid + u * kStateThreads) / (kHeadDim / 4);                                      \
      const int off = min(r, len_ - 1) * static_cast<int>(qk_stride);                                \
      pk[u] = *reinterpret_cast<const f32x4 *>(kg + off);                                            \
      pq[u] = *reinterpret_cast<const f32x4 *>(qg + off);                                            \
    }                                                                                                \
    const size_t wsi = static_cast<size_t>(cid0 + (c)) * p.n_v + j;                                  \
    {                                                                                                \
      const uint4 *tg = reinterpret_cast<const uint4 *>(ws.T + wsi * kChunk * kWsPitch);             \
      const uint4 *pg4 = reinterpret_cast<const uint4 *>(ws.P + wsi * kChunk * kWsPitch);            \
      pt0 = tg[tid];                                                                                 \
      pt1 = tg[tid + kStateThreads];                                                                 \
      pp0 = pg4[tid];                                                                                \
      pp1 = pg4[tid + kStateThreads];                                                                \
    }                                                                                                \
    if (tid < kChunk) {                                                                              \
      pg = ws.gam[wsi * kChunk + tid];                                                               \
      pg_end = ws.gam[wsi * kChunk + kChunk - 1];                                                    \
    }                                                                                                \
    pvv = *reinterpret_cast<const f32x4 *>(p.v + (t0_ + min(v_row, len_ - 1)) * v_stride + j * kHeadDim + \
                                           col_base + 4 * v_c4);                                     \
  } while (0)

// Rows past the chunk's length were loaded from its last row; they are
// zeroed here, where the loaded values are first used, so that the loads
// stay in flight until then.
#define GDN_COMMIT(c)                                                                                \
  do {                                                                                               \
    const int len_ = min(kChunk, L - (c) * kChunk);                                                  \
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};                                                        \
    _Pragma("unroll") for (int u = 0; u < kRowsPer; ++u) {                                           \
      const int idx = tid + u * kStateThreads, r = idx / (kHeadDim / 4), c4 = idx % (kHeadDim / 4);  \
      Op<P>::put4(Kb + r * kPitch128, 4 * c4, r < len_ ? pk[u] : zero4);                             \
      Op<P>::put4(Qb + r * kPitch128, 4 * c4, r < len_ ? pq[u] : zero4);                             \
    }                                                                                                \
    {                                                                                                \
      const int r0 = tid / (kWsPitch / 16), w0 = (tid % (kWsPitch / 16)) * 16;                       \
      const int r1 = r0 + kStateThreads / (kWsPitch / 16);                                           \
      *reinterpret_cast<uint4 *>(Tb + r0 * kPitch64 + w0) = pt0;                                     \
      *reinterpret_cast<uint4 *>(Tb + r1 * kPitch64 + w0) = pt1;                                     \
      *reinterpret_cast<uint4 *>(Pb + r0 * kPitch64 + w0) = pp0;                                     \
      *reinterpret_cast<uint4 *>(Pb + r1 * kPitch64 + w0) = pp1;                                     \
    }                                                                                                \
    if (tid < kChunk) {                                                                              \
      G_s[tid] = expf(static_cast<float>(pg));                                                       \
      ksc_s[tid] = expf(static_cast<float>(pg_end - pg));                                            \
    }                                                                                                \
    *reinterpret_cast<f32x4 *>(Vs + v_row * kLdV + 4 * v_c4) = v_row < len_ ? pvv : zero4;          \
  } while (0)

  if (nchunks > 0) {
    GDN_PREFETCH(0);
    GDN_COMMIT(0);
  }

  for (int ci = 0; ci < nchunks; ++ci) {
    const int t0 = seq0 + ci * kChunk;
    const int len = min(kChunk, L - ci * kChunk);
    block_sync_lds();                        // chunk ci in LDS, St = S at chunk start
    const float g_end = G_s[kChunk - 1];
    // The next chunk's operands are loaded while this one is computed. The
    // last chunk reloads itself, so that every iteration issues and commits
    // the same loads (no loads left in flight across the loop edge).
    const int cnext = min(ci + 1, nchunks - 1);
    GDN_PREFETCH(cnext);

    // X = K S (waves 0-3) or Y = Q S (waves 4-7), rows 16 rt, both column tiles.
    f32x4 XY[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    const uint8_t *Asrc = x_wave ? Kb : Qb;
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 32; ++ks)
      Op<P>::mma2(XY[0], XY[1], frag<P>(Asrc, kPitch128, 16 * rt, 32 * ks), frag<P>(Stb, kPitch128, 0, 32 * ks),
                  frag<P>(Stb, kPitch128, 16, 32 * ks));
    if (x_wave) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f32x4 rv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * rt + acc_row(r);
          rv[r] = Vs[row * kLdV + 16 * ct + acc_col()] - G_s[row] * XY[ct][r];
        }
        put_acc_t<P>(Rtb, kPitch64, 16 * rt, 16 * ct, rv);
      }
    }
    block_sync_lds();

    {  // D = Tm R: tile (rt, wave / 4); D^T and (diag(k~) D)^T to LDS.
      const int ct = wave >> 2;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kChunk / 32; ++ks)
        Op<P>::mma(acc, frag<P>(Tb, kPitch64, 16 * rt, 32 * ks), frag<P>(Rtb, kPitch64, 16 * ct, 32 * ks));
      put_acc_t<P>(Dtb, kPitch64, 16 * rt, 16 * ct, acc);
      f32x4 ds;
#pragma unroll
      for (int r = 0; r < 4; ++r) ds[r] = acc[r] * ksc_s[16 * rt + acc_row(r)];
      put_acc_t<P>(Dsb, kPitch64, 16 * rt, 16 * ct, ds);
    }
    block_sync_lds();

    if (!x_wave) {  // O = s (diag(Gam) Y + P D), rows 16 rt.
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < kChunk / 32; ++ks)
        Op<P>::mma2(acc[0], acc[1], frag<P>(Pb, kPitch64, 16 * rt, 32 * ks), frag<P>(Dtb, kPitch64, 0, 32 * ks),
                    frag<P>(Dtb, kPitch64, 16, 32 * ks));
      // Stage this wave's 16 x 32 rows of O in the (now dead) R^T buffer,
      // then write them out with one 16-byte store per lane (bf16) or two (fp32).
      static_assert(4 * 16 * kLdO * sizeof(float) <= sizeof(Rtb), "O staging must fit the R^T buffer");
      float *Os = reinterpret_cast<float *>(Rtb) + rt * 16 * kLdO;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * rt + acc_row(r);
          Os[acc_row(r) * kLdO + 16 * ct + acc_col()] = scale * (G_s[row] * XY[ct][r] + acc[ct][r]);
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave reads back only its own rows
      const int orow = lane >> 2, oc = 8 * (lane & 3);
      const float *src = Os + orow * kLdO + oc;
      const f32x4 a = *reinterpret_cast<const f32x4 *>(src);
      const f32x4 b = *reinterpret_cast<const f32x4 *>(src + 4);
      if (16 * rt + orow < len) {
        const size_t dst = (t0 + 16 * rt + orow) * v_stride + j * kHeadDim + col_base + oc;
        Act<TA>::store4(o, dst, make_float4(a[0], a[1], a[2], a[3]));
        Act<TA>::store4(o, dst + 4, make_float4(b[0], b[1], b[2], b[3]));
      }
    }
    // S <- Gam_n S + K^T (diag(k~) D); rows 16 wave. K^T is read transposed
    // from the K rows.
    S[0] = S[0] * g_end;
    S[1] = S[1] * g_end;
#pragma unroll
    for (int ks = 0; ks < kChunk / 32; ++ks)
      Op<P>::mma2(S[0], S[1], frag_t<P>(Kb, kPitch128, 16 * wave, 32 * ks), frag<P>(Dsb, kPitch64, 0, 32 * ks),
                  frag<P>(Dsb, kPitch64, 16, 32 * ks));
    block_sync_lds();                        // every read of chunk ci's LDS data is done
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) put_acc_t<P>(Stb, kPitch128, 16 * wave, 16 * ct, S[ct]);
    GDN_COMMIT(cnext);
  }
#undef GDN_PREFETCH
#undef GDN_COMMIT

#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      p.S_out[sbase + static_cast<size_t>(16 * wave + acc_row(r)) * kHeadDim + col_base + 16 * ct + acc_col()] = S[ct][r];
}

}  // namespace

size_t prefill_workspace_bytes(int n_seqs, int n_tokens, int n_v) {
  const int64_t chunks = max_chunks(n_seqs, n_tokens);
  return static_cast<size_t>(chunks) * n_v * (2 * kChunk * kWsPitch + kChunk * sizeof(double));
}

hipError_t launch_prefill(const PrefillParams &p, gdn_dtype act, hipStream_t s) {
  const int64_t chunks = max_chunks(p.n_seqs, p.n_tokens);
  const dim3 grid_local(static_cast<unsigned>(chunks), static_cast<unsigned>(p.n_qk));
  const dim3 grid_state(static_cast<unsigned>(static_cast<int64_t>(p.n_seqs) * p.n_v * (kHeadDim / kSlab)));
  if (act == GDN_BF16) {
    if (p.n_tokens > 0)
      hipLaunchKernelGGL(chunk_local_kernel<Prec::BF16X3>, grid_local, dim3(kLocalThreads), 0, s, p, chunks);
    hipLaunchKernelGGL((chunk_state_kernel<Prec::BF16X3, bf16_t>), grid_state, dim3(kStateThreads), 0, s, p, chunks);
  } else {
    if (p.n_tokens > 0)
      hipLaunchKernelGGL(chunk_local_kernel<Prec::F32>, grid_local, dim3(kLocalThreads), 0, s, p, chunks);
    hipLaunchKernelGGL((chunk_state_kernel<Prec::F32, float>), grid_state, dim3(kStateThreads), 0, s, p, chunks);
  }
  return hipGetLastError();
}

}  // namespace gdn
