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
//  * chunk_local: one block per (chunk, K-head), fully parallel. Writes the
//    chunk's K and Q as ready-to-load MFMA operands, builds K K^T and
//    Q K^T once for the K-head, then for each V-head that uses it (tiled
//    repeat: V-heads h, h + Hqk, ...) applies that head's decays and beta,
//    writes P, and inverts the unit lower-triangular I + A by blocked forward
//    substitution on 16x16 blocks (diagonal blocks by substitution,
//    off-diagonal blocks by fp32 MFMA products), writing Tm and gam.
//  * chunk_state: one block per (sequence, V-head, 32-column slab of S). The
//    value columns of S are independent, so four blocks share a head. It
//    walks the sequence's chunks in order with the fp32 state slab held in
//    MFMA accumulators: [K; Q] S, D = Tm (V - Gam K S), O = s(Gam Q S + P D),
//    S <- Gam_n S + K^T diag(exp(gam_n - gam)) D. The left operands of these
//    products (K, Q, Tm, P) stream from the workspace straight into
//    registers, each reloaded for the next chunk right after its last use;
//    the right operands (S^T, R^T, D^T), V, and the chunk's K rows (from
//    which every wave gathers its K^T fragments) pass through LDS.
// Every product runs at fp32-grade precision: fp32 MFMA for fp32
// activations, three-pass split bf16 MFMA (hi*hi + hi*lo + lo*hi) for bf16
// activations. Operands are split once, when they are written to LDS (or to
// the workspace), never per use. The gated RMSNorm downstream divides by sqrt(mean(o^2) + 1e-6),
// which magnifies absolute errors of low-energy rows of o by up to 1e3, so a
// single bf16 pass is not accurate enough.
//
// Decays: exp is only taken of gam_r - gam_m with m <= r (never positive),
// so nothing overflows; exp(gam) may underflow to 0, which is harmless.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kLocalThreads = 256;        // chunk_local: 4 waves
constexpr int kStateThreads = 512;        // chunk_state: 8 waves
constexpr int kSlab = 32;                 // state columns per chunk_state block
constexpr int kXcds = 8;                  // accelerator complex dies on MI355X
// Row pitches (bytes) of blocked operands in LDS: 128 or 64 contraction
// indices (16 or 8 blocks of 32 bytes) plus 16 bytes to spread LDS banks.
constexpr int kPitch128 = (kHeadDim / 8) * kBlk + 16;   // 528
constexpr int kLdS = kChunk + 1;          // fp32 pitch of the solve's scalar matrices
constexpr int kLdV = kSlab + 4;           // fp32 pitch of the V slab in LDS

// Workspace, all operands in the fragment-major layout:
//   per (chunk, K-head): K rows (64 x 128, 4 x 4 blocks) and Q rows (same): 64 KB
//   per (chunk, V-head): Tm (64 x 64, 4 x 2 blocks) and P (same): 32 KB
//   per (chunk, V-head): gam, 64 fp64
constexpr size_t kKBytes = 16 * kFragBlk;
constexpr size_t kQkBytes = 2 * kKBytes;
constexpr size_t kMatBytes = 8 * kFragBlk;
constexpr size_t kVBytes = 2 * kMatBytes;

struct Workspace {
  uint8_t *qk;
  uint8_t *v;
  double *gam;
};

__host__ __device__ inline Workspace carve(void *ws, int64_t max_chunks, int n_qk, int n_v) {
  Workspace w;
  uint8_t *base = static_cast<uint8_t *>(ws);
  w.qk = base;
  w.v = base + static_cast<size_t>(max_chunks) * n_qk * kQkBytes;
  w.gam = reinterpret_cast<double *>(w.v + static_cast<size_t>(max_chunks) * n_v * kVBytes);
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
// chunk_local: per (chunk, K-head), 4 waves, ~72 KB of LDS (two blocks per CU).
//  1. K rows of the chunk into LDS; Q rows into registers as the A fragments
//     of wave w's row tile, stored to the workspace as they are.
//  2. K operand blocks to the workspace, a whole fragment per lane read out
//     of LDS; wave w computes row tile w of the lower triangles of K K^T and
//     Q K^T.
//  3. For the V-heads that use this K-head (kSolveWaves at a time): decays
//     and beta; L = I + A into LDS and P to the workspace, one fragment
//     block per step spread over all waves; L^-1 by blocked forward
//     substitution in place, one wave per V-head; Tm = L^-1 diag(beta) to
//     the workspace over all waves. Blocks of P and Tm above the diagonal
//     32 x 32 blocks are all zero and are never written or read.
// Fused form: 4 consecutive raw activations as loaded (undecoded, so the load
// can stay in flight until its first use).
template <typename TA> struct RawAct;
template <> struct RawAct<float> {
  using type = float4;
  static __device__ __forceinline__ float4 f4(float4 x) { return x; }
};
template <> struct RawAct<bf16_t> {
  using type = uint2;
  static __device__ __forceinline__ float4 f4(uint2 w) {
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
  }
};

// Fused form: the raw activations of channels c0 .. c0 + 7 (c0 a multiple of
// 8) on rows tl - 3 .. tl of [st_in[n]; qkv rows of sequence n] (0 <= tl <
// L), the inputs of one conv: one 16-byte load per row for bf16, two for
// fp32. They are loaded first and decoded at use, so that every load of a q
// or k row is in flight at once.
template <typename TA> struct Raw8;
template <> struct Raw8<bf16_t> {
  uint4 v[kConvK];
  __device__ __forceinline__ void load(int k, const bf16_t *src) { v[k] = *reinterpret_cast<const uint4 *>(src); }
  __device__ __forceinline__ void get(int k, float4 &a, float4 &b) const {
    a = make_float4(__uint_as_float(v[k].x << 16), __uint_as_float(v[k].x & 0xffff0000u),
                    __uint_as_float(v[k].y << 16), __uint_as_float(v[k].y & 0xffff0000u));
    b = make_float4(__uint_as_float(v[k].z << 16), __uint_as_float(v[k].z & 0xffff0000u),
                    __uint_as_float(v[k].w << 16), __uint_as_float(v[k].w & 0xffff0000u));
  }
};
template <> struct Raw8<float> {
  float4 v[kConvK][2];
  __device__ __forceinline__ void load(int k, const float *src) {
    v[k][0] = *reinterpret_cast<const float4 *>(src);
    v[k][1] = *reinterpret_cast<const float4 *>(src + 4);
  }
  __device__ __forceinline__ void get(int k, float4 &a, float4 &b) const {
    a = v[k][0];
    b = v[k][1];
  }
};
template <typename TA>
__device__ __forceinline__ void load_raw8(const PrefillParams &p, int n, int seq0, int C, int tl, int c0, Raw8<TA> &r) {
  const TA *qkv = static_cast<const TA *>(p.qkv);
  const TA *st = static_cast<const TA *>(p.st_in);
#pragma unroll
  for (int k = 0; k < kConvK; ++k) {
    const int pos = tl - (kConvK - 1) + k;
    const TA *src = pos < 0 ? st + (static_cast<size_t>(n) * (kConvK - 1) + (pos + kConvK - 1)) * C
                            : qkv + static_cast<size_t>(seq0 + pos) * C;
    r.load(k, src + c0);
  }
}
// conv + SiLU of those 8 channels (the same arithmetic as the prep kernel:
// tap 3 meets the current row); w holds their taps.
template <typename TA>
__device__ __forceinline__ void conv_silu8(const Raw8<TA> &r, const float4 *w, f32x4 &ya, f32x4 &yb) {
  float4 xa[kConvK], xb[kConvK];
#pragma unroll
  for (int k = 0; k < kConvK; ++k) r.get(k, xa[k], xb[k]);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float4 we = w[e];
    const float x0 = e < 4 ? (&xa[0].x)[e] : (&xb[0].x)[e - 4];
    const float x1 = e < 4 ? (&xa[1].x)[e] : (&xb[1].x)[e - 4];
    const float x2 = e < 4 ? (&xa[2].x)[e] : (&xb[2].x)[e - 4];
    const float x3 = e < 4 ? (&xa[3].x)[e] : (&xb[3].x)[e - 4];
    y[e] = siluf_(we.x * x0 + we.y * x1 + we.z * x2 + we.w * x3);
  }
  ya = f32x4{y[0], y[1], y[2], y[3]};
  yb = f32x4{y[4], y[5], y[6], y[7]};
}

// Fused form: row tl of q (part 0) or k (part 1) of K-head h, the lane's 32
// channels 32 ks + 8 (lane / 16) .. +7: qk_load issues the raw loads,
// qk_form takes conv + SiLU (taps w of the part's 128 channels) and the L2
// norm over the row's 128 channels (spread over lanes l, l ^ 16, l ^ 32,
// l ^ 48).
template <typename TA>
__device__ __forceinline__ void qk_load(const PrefillParams &p, int n, int seq0, int L, int tl, int part, int h,
                                        Raw8<TA> (&raw)[kHeadDim / 32]) {
  const int C = kHeadDim * (2 * p.n_qk + p.n_v);
  const int cbase = (part * p.n_qk + h) * kHeadDim + 8 * (lane_id() >> 4);
  const int t = min(tl, L - 1);
#pragma unroll
  for (int ks = 0; ks < kHeadDim / 32; ++ks) load_raw8<TA>(p, n, seq0, C, t, cbase + 32 * ks, raw[ks]);
}
template <typename TA>
__device__ __forceinline__ void qk_form(const PrefillParams &p, const Raw8<TA> (&raw)[kHeadDim / 32], const float4 *w,
                                        bool valid, f32x4 (&ya)[kHeadDim / 32], f32x4 (&yb)[kHeadDim / 32]) {
  float ss = 0.f;
#pragma unroll
  for (int ks = 0; ks < kHeadDim / 32; ++ks) {
    conv_silu8<TA>(raw[ks], w + 32 * ks + 8 * (lane_id() >> 4), ya[ks], yb[ks]);
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += ya[ks][e] * ya[ks][e] + yb[ks][e] * yb[ks][e];
  }
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  const float inv = valid ? l2_inv(ss, p.l2_eps, p.l2_mode == GDN_L2_RSQRT) : 0.f;
#pragma unroll
  for (int ks = 0; ks < kHeadDim / 32; ++ks) {
    ya[ks] *= inv;
    yb[ks] *= inv;
  }
}

constexpr int kSolveWaves = 3;
constexpr int kTri = kChunk * (kChunk + 1) / 2;   // packed lower triangle incl. diagonal

__device__ __forceinline__ int tri(int r, int m) { return r * (r + 1) / 2 + m; }

// Orders this wave's earlier LDS accesses before its later ones.
__device__ __forceinline__ void wave_sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// LDS of one chunk_local unit, carved from one byte array (so that a block
// of the sequential kernel can hold two units):
//   buf: K as blocked operand rows first; then the solving waves' fp32
//        matrices (L, overwritten in place by L^-1) reuse the bytes
//   Wtap (fused): conv taps of the K-head's q and k channels
//   gam_s, bet_s: per solving wave; Gk, Gq: K K^T and Q K^T, lower
//   triangles; Tsc: per solving wave, an off-diagonal block in transit
struct LocalLds {
  static constexpr int kKbBytes = kChunk * kPitch128;
  static constexpr int kLxBytes = kSolveWaves * kChunk * kLdS * 4;
  static constexpr size_t kBuf = 0;
  static constexpr size_t kWtap = (kKbBytes > kLxBytes ? kKbBytes : kLxBytes);
  static constexpr size_t kGam = kWtap + 2 * kHeadDim * sizeof(float4);
  static constexpr size_t kGk = kGam + kSolveWaves * kChunk * sizeof(double);
  static constexpr size_t kGq = kGk + kTri * sizeof(float);
  static constexpr size_t kTsc = kGq + kTri * sizeof(float);
  static constexpr size_t kBet = kTsc + kSolveWaves * 16 * 17 * sizeof(float);
  static constexpr size_t kBytes = kBet + kSolveWaves * kChunk * sizeof(float);
};
static_assert(LocalLds::kWtap % 16 == 0 && LocalLds::kGam % 8 == 0, "LDS carve alignment");

// One (chunk, K-head) unit of chunk_local: unit cid = chunk ci of sequence n
// (a valid one), K-head h, on 4 waves (tid 0 .. 255 of them) with the LDS at
// smem. Every barrier is taken by the whole block, the same number of times
// whatever the unit, so two units can run side by side in one block. live =
// false runs a unit without any global store (a block's second slot with no
// unit of its own).
template <Prec P, typename TA, bool kFused>
__device__ __forceinline__ void local_unit(const PrefillParams &p, int64_t max_chunks, int cid, int n, int ci, int h,
                                           uint8_t *smem, int tid, bool live) {
  using Frag = typename Op<P>::Frag;
  uint8_t *buf = smem + LocalLds::kBuf;
  float4 *Wtap = reinterpret_cast<float4 *>(smem + LocalLds::kWtap);
  double (*gam_s)[kChunk] = reinterpret_cast<double (*)[kChunk]>(smem + LocalLds::kGam);
  float *Gk = reinterpret_cast<float *>(smem + LocalLds::kGk);
  float *Gq = reinterpret_cast<float *>(smem + LocalLds::kGq);
  float (*Tsc)[16 * 17] = reinterpret_cast<float (*)[16 * 17]>(smem + LocalLds::kTsc);
  float (*bet_s)[kChunk] = reinterpret_cast<float (*)[kChunk]>(smem + LocalLds::kBet);
  uint8_t *Kb = buf;

  const int wave = tid / kWave;
  const int lane = lane_id();
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  const int t0 = seq0 + ci * kChunk;
  const int len = min(kChunk, L - ci * kChunk);
  const Workspace ws = carve(p.ws, max_chunks, p.n_qk, p.n_v);
  const size_t qk_stride = static_cast<size_t>(p.n_qk) * kHeadDim;
  const float *kg = kFused ? nullptr : p.k + t0 * qk_stride + h * kHeadDim;
  const float *qg = kFused ? nullptr : p.q + t0 * qk_stride + h * kHeadDim;
  uint8_t *wk = ws.qk + (static_cast<size_t>(cid) * p.n_qk + h) * kQkBytes;   // K rows, Q rows
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // Every global load of the block (K and Q rows, the gate inputs of the
  // first round of V-heads) is issued before its first workspace store:
  // once stores and loads are both in flight, the compiler's memory waits
  // also wait for the stores to complete.
  const int nvh = p.n_v / p.n_qk;
  // Gates of V-head h + u Hqk for row lane of the chunk (rows past len repeat
  // the last row and are masked where used), as the prep kernel forms them:
  // the raw inputs are loaded by load_gates and turned into (g, beta) by
  // form_gates at first use, so that the loads stay in flight meanwhile.
  using RawGate = std::conditional_t<kFused && std::is_same<TA, bf16_t>::value, uint16_t, float>;
  auto load_gates = [&](int u, RawGate &gr, RawGate &br) {
    const int j = h + u * p.n_qk;
    const size_t e = static_cast<size_t>(t0 + min(lane, len - 1)) * p.n_v + j;
    if constexpr (kFused) {
      br = static_cast<const RawGate *>(p.bl)[e];
      gr = static_cast<const RawGate *>(p.al)[e];
    } else {
      br = p.beta[e];
      gr = p.g[e];
    }
  };
  auto form_gates = [&](int u, RawGate gr, RawGate br, float &gv, float &bv) {
    if constexpr (kFused) {
      const int j = h + u * p.n_qk;
      float b_logit, a_logit;
      if constexpr (std::is_same<RawGate, uint16_t>::value) {
        b_logit = __uint_as_float(static_cast<uint32_t>(br) << 16);
        a_logit = __uint_as_float(static_cast<uint32_t>(gr) << 16);
      } else {
        b_logit = br;
        a_logit = gr;
      }
      bv = sigmoidf_(b_logit);
      gv = -expf(p.A_log[j]) * softplusf_(a_logit + p.dt_bias[j]);
    } else {
      bv = br;
      gv = gr;
    }
  };
  RawGate g_first{}, b_first{};   // wave w < min(nvh, kSolveWaves): V-head h + w Hqk

  // Q rows of this wave's row tile as A fragments (rows >= len are zero);
  // they are also the Q operand blocks (wave, ks) of the workspace.
  const int rt = wave;
  const int qrow = 16 * rt + (lane & 15);
  Frag fq[kHeadDim / 32];
  if constexpr (kFused) {
    // k and q of row qrow from the raw rows; k goes to LDS (blocked operand
    // rows, as below), q stays in this lane's A-fragment slots. The conv
    // taps of the K-head's q and k channels go to LDS; the raw loads of
    // both rows (bf16; fp32 would need twice the registers: one row at a
    // time) are issued before any is used.
    constexpr bool kBoth = sizeof(TA) == 2;
    const float4 wtap = reinterpret_cast<const float4 *>(p.conv_w)[((tid >> 7) * p.n_qk + h) * kHeadDim + (tid & 127)];
    Raw8<TA> rk[kHeadDim / 32], rq[kHeadDim / 32];
    qk_load<TA>(p, n, seq0, L, ci * kChunk + qrow, 1, h, rk);
    if constexpr (kBoth) qk_load<TA>(p, n, seq0, L, ci * kChunk + qrow, 0, h, rq);
    if (wave < min(nvh, kSolveWaves)) load_gates(wave, g_first, b_first);
    Wtap[tid] = wtap;   // q taps at 0, k taps at kHeadDim
    block_sync_lds();
    const bool valid = qrow < len;
    f32x4 ya[kHeadDim / 32], yb[kHeadDim / 32];
    qk_form<TA>(p, rk, Wtap + kHeadDim, valid, ya, yb);
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 32; ++ks) {
      const int c = 32 * ks + 8 * (lane >> 4);
      Op<P>::put4(Kb + qrow * kPitch128, c, ya[ks]);
      Op<P>::put4(Kb + qrow * kPitch128, c + 4, yb[ks]);
    }
    if constexpr (!kBoth) qk_load<TA>(p, n, seq0, L, ci * kChunk + qrow, 0, h, rq);
    qk_form<TA>(p, rq, Wtap, valid, ya, yb);
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 32; ++ks) fq[ks] = make_frag<P>(ya[ks], yb[ks]);
  } else {
    // K rows -> blocked operand rows in LDS; rows >= len are zero.
    constexpr int kPer = kChunk * (kHeadDim / 4) / kLocalThreads;
    f32x4 kb4[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = tid + u * kLocalThreads, r = idx / (kHeadDim / 4), c4 = idx % (kHeadDim / 4);
      kb4[u] = *reinterpret_cast<const f32x4 *>(kg + min(r, len - 1) * qk_stride + 4 * c4);
    }
    const float *qp = qg + min(qrow, len - 1) * qk_stride + 8 * (lane >> 4);
    f32x4 qa[kHeadDim / 32], qb[kHeadDim / 32];
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 32; ++ks) {
      qa[ks] = *reinterpret_cast<const f32x4 *>(qp + 32 * ks);
      qb[ks] = *reinterpret_cast<const f32x4 *>(qp + 32 * ks + 4);
    }
    if (wave < min(nvh, kSolveWaves)) load_gates(wave, g_first, b_first);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = tid + u * kLocalThreads, r = idx / (kHeadDim / 4), c4 = idx % (kHeadDim / 4);
      Op<P>::put4(Kb + r * kPitch128, 4 * c4, r < len ? kb4[u] : zero4);
    }
    const bool qvalid = qrow < len;
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 32; ++ks)
      fq[ks] = make_frag<P>(qvalid ? qa[ks] : zero4, qvalid ? qb[ks] : zero4);
  }
  // The first round's gates are formed before the first store (a wait for
  // their loads after it would also wait for the stores).
  float g_first_v = 0.f, b_first_v = 0.f;
  if (wave < min(nvh, kSolveWaves)) form_gates(wave, g_first, b_first, g_first_v, b_first_v);
  if (live)
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 32; ++ks) FragIO<P>::store(wk + kKBytes, kHeadDim / 32, rt, ks, fq[ks]);
  block_sync_lds();

  // K rows (4 x 4 blocks) to the workspace, read out of LDS a whole
  // fragment at a time: wave w stores blocks w, w + 4, ..
  if (live)
#pragma unroll
    for (int b = wave; b < 16; b += 4)
      FragIO<P>::store(wk, kHeadDim / 32, b >> 2, b & 3, frag<P>(Kb, kPitch128, 16 * (b >> 2), 32 * (b & 3)));
  // Row tile rt of the lower triangles of K K^T and Q K^T.
  for (int ct = 0; ct <= rt; ++ct) {
    f32x4 ak = zero4, aq = zero4;
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 32; ++ks) {
      const Frag b = frag<P>(Kb, kPitch128, ct * 16, ks * 32);
      Op<P>::mma(ak, frag<P>(Kb, kPitch128, rt * 16, ks * 32), b);
      Op<P>::mma(aq, fq[ks], b);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * rt + acc_row(r), col = 16 * ct + acc_col();
      if (col <= row) {
        Gk[tri(row, col)] = ak[r];
        Gq[tri(row, col)] = aq[r];
      }
    }
  }
  block_sync_lds();   // K is dead from here: buf becomes the solving waves' matrices

  // The 16 x 32 blocks (rt, ks) of a 64 x 64 lower-triangular operand that
  // are not all zero (blocks (0, 1) and (1, 1) are): block bl = 0 .. 5 is
  // (0, 0), (1, 0), (2, 0), (2, 1), (3, 0), (3, 1), formed arithmetically (an
  // indexed table would be read from global memory).
  constexpr int kLowBlocks = 6;
  auto low_rt = [](int bl) { return bl < 2 ? bl : 2 + ((bl - 2) >> 1); };
  auto low_ks = [](int bl) { return bl < 2 ? 0 : (bl & 1); };

  for (int u0 = 0; u0 < nvh; u0 += kSolveWaves) {
    const int nu = min(kSolveWaves, nvh - u0);   // V-heads of this round, slot s = head u0 + s
    if (u0 > 0) block_sync_lds();                // the previous round's readers are done
    // Cumulative log-decay (0 past len, so gam stays at its last value) and
    // beta, one wave per V-head. gam reaches a few hundred inside a chunk and
    // only its differences gam_r - gam_m are used: in fp32 they would lose
    // ~|gam| * 6e-8 to cancellation, so the scan and the differences are fp64.
    if (wave < nu) {
      const int j = h + (u0 + wave) * p.n_qk;
      float gv = g_first_v, bv = b_first_v;
      if (u0 > 0) {
        RawGate graw, braw;
        load_gates(u0 + wave, graw, braw);
        form_gates(u0 + wave, graw, braw, gv, bv);
      }
      const double gr = lane < len ? static_cast<double>(gv) : 0.0;
      const float br = lane < len ? bv : 0.f;
      const double gm = wave_inclusive_scan_d(gr);
      gam_s[wave][lane] = gm;
      bet_s[wave][lane] = br;
      if (live) ws.gam[(static_cast<size_t>(cid) * p.n_v + j) * kChunk + lane] = gm;
    }
    block_sync_lds();

    // L = I + A into LDS and P to the workspace, one fragment block per step,
    // spread over all waves: lane l owns row 16 rt + l % 16, columns
    // 32 ks + 8 (l / 16) + 0..7 of the block.
    for (int item = wave; item < nu * kLowBlocks; item += kLocalThreads / kWave) {
      const int s = item / kLowBlocks, bl = item % kLowBlocks;
      const int brt = low_rt(bl), bks = low_ks(bl);
      const int j = h + (u0 + s) * p.n_qk;
      float *Lx = reinterpret_cast<float *>(buf) + s * kChunk * kLdS;
      const double *gam = gam_s[s];
      const int r = 16 * brt + (lane & 15), m0 = 32 * bks + 8 * (lane >> 4);
      const double gr = gam[r];
      const float br = bet_s[s][r];
      // Every operand of the lane's 8 entries is read first, above the
      // diagonal too (in-bounds values that are then discarded), so that the
      // reads overlap. gam_r - gam_m <= 0 for m <= r; the clamp only keeps the
      // discarded entries finite.
      double gm[8];
      float qk[8], kk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        gm[e] = gam[m0 + e];
        qk[e] = Gq[tri(r, m0 + e)];
        kk[e] = Gk[tri(r, m0 + e)];
      }
      // Decays by the hardware exp (exp2 of x log2 e): for x <= 0 its relative
      // error is about |x| 2^-24, and the factors it loses accuracy on (large
      // |x|) are far below the others.
      f32x4 pa, pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = m0 + e;
        const float dec = __expf(fminf(static_cast<float>(gr - gm[e]), 0.f));
        const float pv = m <= r ? dec * qk[e] : 0.f;
        const float lv = m < r ? br * dec * kk[e] : (m == r ? 1.f : 0.f);
        Lx[r * kLdS + m] = lv;
        if (e < 4) pa[e] = pv; else pb[e - 4] = pv;
      }
      uint8_t *wv = ws.v + (static_cast<size_t>(cid) * p.n_v + j) * kVBytes;   // Tm, then P
      if (live) FragIO<P>::store(wv + kMatBytes, kChunk / 32, brt, bks, make_frag<P>(pa, pb));
    }
    block_sync_lds();

    if (wave < nu) {
      float *Lx = reinterpret_cast<float *>(buf) + wave * kChunk * kLdS;
      // Diagonal blocks X_bb = L_bb^-1 by forward substitution: lane 16 b + c
      // owns column c of block b and writes it over L_bb.
      {
        const int b = lane >> 4, c = lane & 15;
        const float *Lb = Lx + (b * 16) * kLdS + b * 16;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float acc = r == c ? 1.f : 0.f;
#pragma unroll
          for (int m = 0; m < r; ++m) acc -= Lb[r * kLdS + m] * x[m];
          x[r] = acc;
        }
        wave_sync_lds();
#pragma unroll
        for (int r = 0; r < 16; ++r) Lx[(b * 16 + r) * kLdS + b * 16 + c] = x[r];
      }
      wave_sync_lds();

      // Off-diagonal blocks, in place: for block row i and j = 0 .. i-1 in
      // order, X_ij = -X_ii * sum_{k=j}^{i-1} L_ik X_kj. Block (i, k) still
      // holds L_ik for k >= j (only blocks left of j were overwritten), and
      // blocks of rows above i already hold X.
      float *ts = Tsc[wave];
      for (int bi = 1; bi < 4; ++bi) {
        for (int bj = 0; bj < bi; ++bj) {
          f32x4 acc = zero4;
          for (int bk = bj; bk < bi; ++bk) {
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
              const float a = Lx[(bi * 16 + (lane & 15)) * kLdS + bk * 16 + 4 * k4 + (lane >> 4)];
              const float b = Lx[(bk * 16 + 4 * k4 + (lane >> 4)) * kLdS + bj * 16 + (lane & 15)];
              acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) ts[acc_row(r) * 17 + acc_col()] = acc[r];
          wave_sync_lds();
          f32x4 x = zero4;
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) {
            const float a = Lx[(bi * 16 + (lane & 15)) * kLdS + bi * 16 + 4 * k4 + (lane >> 4)];
            const float b = ts[(4 * k4 + (lane >> 4)) * 17 + (lane & 15)];
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, x, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) Lx[(bi * 16 + acc_row(r)) * kLdS + bj * 16 + acc_col()] = -x[r];
          wave_sync_lds();
        }
      }
    }
    block_sync_lds();

    // Tm = X diag(beta) (lower triangle) to the workspace, one fragment block
    // per step over all waves.
    for (int item = wave; item < nu * kLowBlocks; item += kLocalThreads / kWave) {
      const int s = item / kLowBlocks, bl = item % kLowBlocks;
      const int brt = low_rt(bl), bks = low_ks(bl);
      const int j = h + (u0 + s) * p.n_qk;
      const float *Lx = reinterpret_cast<const float *>(buf) + s * kChunk * kLdS;
      const float *bet = bet_s[s];
      const int r = 16 * brt + (lane & 15), m0 = 32 * bks + 8 * (lane >> 4);
      float xv[8], bv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {   // read first (in bounds above the diagonal too), then select
        xv[e] = Lx[r * kLdS + m0 + e];
        bv[e] = bet[m0 + e];
      }
      f32x4 ta, tb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float tv = m0 + e <= r ? xv[e] * bv[e] : 0.f;
        if (e < 4) ta[e] = tv; else tb[e - 4] = tv;
      }
      uint8_t *wv = ws.v + (static_cast<size_t>(cid) * p.n_v + j) * kVBytes;
      if (live) FragIO<P>::store(wv, kChunk / 32, brt, bks, make_frag<P>(ta, tb));
    }
  }
}

template <Prec P, typename TA, bool kFused>
__global__ __launch_bounds__(kLocalThreads) void chunk_local_kernel(PrefillParams p, int64_t max_chunks) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LocalLds::kBytes];
  const int h = blockIdx.y;
  int n, ci;
  if (!find_unit(p.cu, p.n_seqs, blockIdx.x, kChunk, 0, &n, &ci)) return;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  if (seq0 < 0 || L < 0 || seq0 + L > p.n_tokens) return;
  local_unit<P, TA, kFused>(p, max_chunks, blockIdx.x, n, ci, h, smem, threadIdx.x, true);
  // Folded norm: the ready counters of this chunk's V-heads start at zero
  // (the next launch sees them at zero: a kernel boundary orders the two).
  if constexpr (kFused) {
    const int nvh = p.n_v / p.n_qk;
    if (p.fold_blocks > 0)
      for (int u = threadIdx.x; u < nvh; u += kLocalThreads)
        p.ready[(static_cast<size_t>(blockIdx.x) * p.n_v + h + u * p.n_qk) * kReadyStride] = 0u;
  }
}

// ---------------------------------------------------------------------------
// Folded gated RMSNorm and new conv state (fused form, when chunk_state's
// slab blocks leave CUs idle). A row's norm needs all 128 columns of o, which
// four slab blocks produce. Instead of a launch of its own after chunk_state,
// extra "norm blocks" of the same launch, on the idle CUs, form y chunk by
// chunk as the slab blocks finish:
//  * each y-wave of a slab block stores its o rows of chunk c, and at the top
//    of the iteration after next (its loads of the iteration between must
//    land there anyway) waits for its memory operations and adds 1 to the
//    ready counter of (chunk, V-head);
//  * the norm wave that owns a quarter (16 rows) of the pair polls the
//    counter until it reads 16 (4 slab blocks x 4 y-waves), then normalises
//    those rows exactly as the norm kernel does.
// Publication across XCDs (each has its own L2): o is written with
// agent-scope atomic stores and read with agent-scope atomic loads, which
// the compiler emits as device-coherent accesses (sc1) with no cache
// maintenance; the counter is an agent-scope atomic. The writer's wait for
// all of its memory operations before the add orders its o stores before
// the add, and the reader issues its o loads only after its counter load
// returned 16. This is the ordering a release/acquire pair gives, minus the
// whole-L2 write-back and invalidate that such a pair emits on this chip
// for plain accesses (measured: 1.8 ms instead of 0.24 ms per fused step).
// z and y go through with non-temporal accesses: kept out of L2, where the
// slab blocks share their K, Q, Tm and P operands (16 us per step).
// Counters sit 128 bytes apart: polls and adds of neighbouring pairs on one
// line slowed the step by tens of us.
// Norm blocks only ever wait for slab blocks, never the reverse, so the
// launch drains in whatever order its blocks are placed. A wave's items lie
// G / (4 Hv) chunks apart (G = its launch's norm waves), so it waits for any
// one of them at most about as long as the slab blocks take for that many
// chunks, well under a millisecond however long the sequences. Each wait is
// bounded (about a second); once one runs out the wave waits no more, and
// rows whose counter is not complete (only cu_seqlens outside the contract
// leave one short) get NaN.
// The same norm waves write the new conv states: the V channels of head j
// once the counter of the sequence's first chunk of j is full (the four slab
// blocks of j read the old state only before that chunk, so the update can
// be in place), the q and k channels of K-head h (read only by chunk_local,
// in the launch before) with those of V-head h, and whole states of
// sequences without tokens (which nothing else reads) first.
constexpr uint32_t kFoldReady = 16;       // 4 slab blocks x 4 y-waves
constexpr int kFoldSleep = 48;            // s_sleep units (64 cycles) between polls
constexpr int kFoldSpins = 1 << 20;       // polls per item, each a load and a sleep

__device__ __forceinline__ void fold_put4(bf16_t *o, size_t i, f32x4 a) {
  const uint64_t w = static_cast<uint64_t>(f32_to_bf16(a[0])) | (static_cast<uint64_t>(f32_to_bf16(a[1])) << 16) |
                     (static_cast<uint64_t>(f32_to_bf16(a[2])) << 32) |
                     (static_cast<uint64_t>(f32_to_bf16(a[3])) << 48);
  __hip_atomic_store(reinterpret_cast<uint64_t *>(o + i), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fold_put4(float *o, size_t i, f32x4 a) {
  uint64_t *d = reinterpret_cast<uint64_t *>(o + i);
  __hip_atomic_store(d, (static_cast<uint64_t>(__float_as_uint(a[1])) << 32) | __float_as_uint(a[0]),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(d + 1, (static_cast<uint64_t>(__float_as_uint(a[3])) << 32) | __float_as_uint(a[2]),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t fold_ld64(const void *p) {
  return __hip_atomic_load(reinterpret_cast<uint64_t *>(const_cast<void *>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 bf16x4_f4(uint32_t x, uint32_t y) {
  return make_float4(__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u), __uint_as_float(y << 16),
                     __uint_as_float(y & 0xffff0000u));
}
__device__ __forceinline__ void fold_get8(const bf16_t *o, size_t i, float4 &a, float4 &b) {
  const uint64_t u = fold_ld64(o + i), v = fold_ld64(o + i + 4);
  a = bf16x4_f4(static_cast<uint32_t>(u), static_cast<uint32_t>(u >> 32));
  b = bf16x4_f4(static_cast<uint32_t>(v), static_cast<uint32_t>(v >> 32));
}
__device__ __forceinline__ void fold_get8(const float *o, size_t i, float4 &a, float4 &b) {
  const uint64_t u0 = fold_ld64(o + i), u1 = fold_ld64(o + i + 2), u2 = fold_ld64(o + i + 4), u3 = fold_ld64(o + i + 6);
  a = make_float4(__uint_as_float(static_cast<uint32_t>(u0)), __uint_as_float(static_cast<uint32_t>(u0 >> 32)),
                  __uint_as_float(static_cast<uint32_t>(u1)), __uint_as_float(static_cast<uint32_t>(u1 >> 32)));
  b = make_float4(__uint_as_float(static_cast<uint32_t>(u2)), __uint_as_float(static_cast<uint32_t>(u2 >> 32)),
                  __uint_as_float(static_cast<uint32_t>(u3)), __uint_as_float(static_cast<uint32_t>(u3 >> 32)));
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void fold_in8(const bf16_t *z, size_t i, float4 &a, float4 &b) {
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(z + i));
  a = bf16x4_f4(w[0], w[1]);
  b = bf16x4_f4(w[2], w[3]);
}
__device__ __forceinline__ void fold_in8(const float *z, size_t i, float4 &a, float4 &b) {
  const f32x4 u = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(z + i));
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(z + i + 4));
  a = make_float4(u[0], u[1], u[2], u[3]);
  b = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void fold_out8(bf16_t *y, size_t i, float4 a, float4 b) {
  const u32x4 w = {static_cast<uint32_t>(f32_to_bf16(a.x)) | (static_cast<uint32_t>(f32_to_bf16(a.y)) << 16),
                   static_cast<uint32_t>(f32_to_bf16(a.z)) | (static_cast<uint32_t>(f32_to_bf16(a.w)) << 16),
                   static_cast<uint32_t>(f32_to_bf16(b.x)) | (static_cast<uint32_t>(f32_to_bf16(b.y)) << 16),
                   static_cast<uint32_t>(f32_to_bf16(b.z)) | (static_cast<uint32_t>(f32_to_bf16(b.w)) << 16)};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(y + i));
}
__device__ __forceinline__ void fold_out8(float *y, size_t i, float4 a, float4 b) {
  const f32x4 u = {a.x, a.y, a.z, a.w}, v = {b.x, b.y, b.z, b.w};
  __builtin_nontemporal_store(u, reinterpret_cast<f32x4 *>(y + i));
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(y + i + 4));
}

// One norm block (block fb of p.fold_blocks). Work items are 16-row quarters
// of (chunk, V-head) pairs, so that the pairs of the last chunk, ready only
// as the slab blocks end, spread over four times as many waves. Wave w owns
// items i = g, g + G, ... with g = w * fold_blocks + fb and G the number of
// norm waves (consecutive items on different CUs). 16 lanes per row (8
// values each), 4 rows per pass, all 16 rows' loads in flight together.
template <typename TA>
__device__ __forceinline__ void fold_norm(const PrefillParams &p, int64_t max_chunks, int fb) {
  constexpr int kWaves = kStateThreads / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int sub = lane & 15, r4 = lane >> 4;
  const int64_t g = static_cast<int64_t>(wave) * p.fold_blocks + fb;
  const int64_t G = static_cast<int64_t>(p.fold_blocks) * kWaves;
  const size_t stride = static_cast<size_t>(p.n_v) * kHeadDim;
  const TA *o = static_cast<const TA *>(p.o);
  const TA *z = static_cast<const TA *>(p.z);
  TA *y = static_cast<TA *>(p.y);
  ConvStateParams cp;
  cp.cu = p.cu;
  cp.n_seqs = p.n_seqs;
  cp.n_tokens = p.n_tokens;
  cp.C = kHeadDim * (2 * p.n_qk + p.n_v);
  cp.qkv = p.qkv;
  cp.st_in = p.st_in;
  cp.st_out = p.st_out;
  for (int64_t n = g; n < p.n_seqs; n += G)
    if (p.cu[n + 1] == p.cu[n])
      for (int c = 2 * lane; c < cp.C; c += 2 * kWave) conv_state_pair<TA>(cp, static_cast<int>(n), c);

  const float4 w0 = *reinterpret_cast<const float4 *>(p.norm_w + 8 * sub);
  const float4 w1 = *reinterpret_cast<const float4 *>(p.norm_w + 8 * sub + 4);
  const int64_t items = max_chunks * p.n_v * 4;
  bool waiting = true;   // false once a wait has run out
  for (int64_t it = g; it < items; it += G) {
    const int64_t t = it >> 2;
    const int rb = 16 * static_cast<int>(it & 3);
    const int cid = static_cast<int>(t / p.n_v), j = static_cast<int>(t % p.n_v);
    int n, ci;
    if (!find_unit(p.cu, p.n_seqs, cid, kChunk, 0, &n, &ci)) break;   // every later item is past the last chunk
    const int seq0 = p.cu[n];
    const int L = p.cu[n + 1] - seq0;
    if (seq0 < 0 || L < 0 || seq0 + L > p.n_tokens) continue;   // skipped by the slab blocks too
    const int t0 = seq0 + ci * kChunk;
    const int len = min(kChunk, L - ci * kChunk);
    if (rb >= len) continue;
    const uint32_t *rdy = p.ready + t * kReadyStride;
    uint32_t cnt = __hip_atomic_load(rdy, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // readfirstlane returns int: back to the counter's unsigned type.
    for (int spins = 0; waiting && static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(cnt)) < kFoldReady; ++spins) {
      if (spins == kFoldSpins) {
        waiting = false;
        break;
      }
      __builtin_amdgcn_s_sleep(kFoldSleep);
      cnt = __hip_atomic_load(rdy, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const bool ok = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(cnt)) >= kFoldReady;
    float4 o0[4], o1[4], z0[4], z1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = min(rb + 4 * u + r4, len - 1);
      const size_t i = static_cast<size_t>(t0 + row) * stride + static_cast<size_t>(j) * kHeadDim + 8 * sub;
      fold_get8(o, i, o0[u], o1[u]);
      fold_in8(z, i, z0[u], z1[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = rb + 4 * u + r4;
      float ss = o0[u].x * o0[u].x + o0[u].y * o0[u].y + o0[u].z * o0[u].z + o0[u].w * o0[u].w +
                 o1[u].x * o1[u].x + o1[u].y * o1[u].y + o1[u].z * o1[u].z + o1[u].w * o1[u].w;
      ss = row16_sum(ss);
      const float inv = ok ? 1.0f / sqrtf(ss * (1.0f / kHeadDim) + p.norm_eps) : __builtin_nanf("");
      float4 y0, y1;
      y0.x = o0[u].x * inv * w0.x * siluf_(z0[u].x);
      y0.y = o0[u].y * inv * w0.y * siluf_(z0[u].y);
      y0.z = o0[u].z * inv * w0.z * siluf_(z0[u].z);
      y0.w = o0[u].w * inv * w0.w * siluf_(z0[u].w);
      y1.x = o1[u].x * inv * w1.x * siluf_(z1[u].x);
      y1.y = o1[u].y * inv * w1.y * siluf_(z1[u].y);
      y1.z = o1[u].z * inv * w1.z * siluf_(z1[u].z);
      y1.w = o1[u].w * inv * w1.w * siluf_(z1[u].w);
      if (row < len)
        fold_out8(y, static_cast<size_t>(t0 + row) * stride + static_cast<size_t>(j) * kHeadDim + 8 * sub, y0, y1);
    }
    if (ok && ci == 0 && rb == 0) {
      conv_state_pair<TA>(cp, n, kHeadDim * (2 * p.n_qk + j) + 2 * lane);
      if (j < p.n_qk) {
        conv_state_pair<TA>(cp, n, kHeadDim * j + 2 * lane);
        conv_state_pair<TA>(cp, n, kHeadDim * (p.n_qk + j) + 2 * lane);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Right operands of chunk_state live in LDS in the fragment-major layout of
// the MFMA B operand: one 2 KB block per 32 x 16 (k x column) tile, lane l's
// 16 bytes at l * 16 of each 1 KB plane (BF16X3: plane 0 = hi, plane 1 =
// lo; F32: plane 0 = indices 0..3 of the lane's 8, plane 1 = indices 4..7).
// A wave reads a fragment as two linear 1 KB reads, free of LDS bank
// conflicts (gfx950 LDS: 64 banks of 4 bytes).
constexpr int kLdsBlk = 2048;
constexpr int kLdOs = kSlab + 4;         // fp32 pitch of the O staging rows

template <Prec P> __device__ __forceinline__ typename Op<P>::Frag lds_frag(const uint8_t *buf, int blk);
template <> __device__ __forceinline__ Op<Prec::F32>::Frag lds_frag<Prec::F32>(const uint8_t *buf, int blk) {
  const uint8_t *b = buf + blk * kLdsBlk + lane_id() * 16;
  Op<Prec::F32>::Frag f;
  f.a = *reinterpret_cast<const f32x4 *>(b);
  f.b = *reinterpret_cast<const f32x4 *>(b + kLdsBlk / 2);
  return f;
}
template <> __device__ __forceinline__ Op<Prec::BF16X3>::Frag lds_frag<Prec::BF16X3>(const uint8_t *buf, int blk) {
  const uint8_t *b = buf + blk * kLdsBlk + lane_id() * 16;
  Op<Prec::BF16X3>::Frag f;
  f.hi = *reinterpret_cast<const bf16x8 *>(b);
  f.lo = *reinterpret_cast<const bf16x8 *>(b + kLdsBlk / 2);
  return f;
}

// Store contraction indices k0 .. k0+3 (k0 % 4 == 0) of column c of a right
// operand with KS contraction steps of 32 (one accumulator's four values).
template <Prec P> __device__ __forceinline__ void lds_put4(uint8_t *buf, int KS, int k0, int c, f32x4 x);
template <> __device__ __forceinline__ void lds_put4<Prec::F32>(uint8_t *buf, int KS, int k0, int c, f32x4 x) {
  const int blk = (c >> 4) * KS + (k0 >> 5);
  const int ln = 16 * ((k0 & 31) >> 3) + (c & 15);
  *reinterpret_cast<f32x4 *>(buf + blk * kLdsBlk + ((k0 & 4) ? kLdsBlk / 2 : 0) + ln * 16) = x;
}
template <> __device__ __forceinline__ void lds_put4<Prec::BF16X3>(uint8_t *buf, int KS, int k0, int c, f32x4 x) {
  const int blk = (c >> 4) * KS + (k0 >> 5);
  const int ln = 16 * ((k0 & 31) >> 3) + (c & 15);
  bf16x4 hi, lo;
  split4(x, hi, lo);
  uint8_t *b = buf + blk * kLdsBlk + ln * 16 + (k0 & 7) * 2;
  *reinterpret_cast<bf16x4 *>(b) = hi;
  *reinterpret_cast<bf16x4 *>(b + kLdsBlk / 2) = lo;
}

// K rows of the current chunk in LDS, for the transposed (K^T) fragments of
// the state update: BF16X3 keeps the hi and lo planes as bf16, F32 one fp32
// plane, row-major (token rows, key index contiguous).
//
// BF16X3 reads its K^T fragments with the gfx950 transpose read
// ds_read_b64_tr_b16: within each group of 16 lanes, output lane j receives
// element j & 3 of the 4 16-bit values that lanes (j >> 2) + 4 e (e = 0..3)
// address (checked on the GPU). Lane s of group g pointing at row
// t0 + (s >> 2), columns i0 + 4 (s & 3) .. +3 therefore yields
// K[t0 + e][i0 + s] for e = 0..3: four consecutive tokens of one key index,
// half of an A fragment of K^T. Rows of kLdKt = 144 elements (288 bytes)
// keep the 16-byte stores aligned and put 4 consecutive rows of a read on
// disjoint banks.
constexpr int kLdKt = kHeadDim + 16;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 lds_read_tr16(const __bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(const_cast<__bf16 *>(p)));
}

template <Prec P> struct KtLds;
template <> struct KtLds<Prec::BF16X3> {
  static constexpr int kBytes = 2 * kChunk * kLdKt * 2;
  // Store this lane's fragment (rt, ks) of K rows: row 16 rt + l % 16,
  // indices 32 ks + 8 (l / 16) .. +7.
  static __device__ __forceinline__ void put(uint8_t *buf, int rt, int ks, const Op<Prec::BF16X3>::Frag &f) {
    const int l = lane_id();
    __bf16 *hi = reinterpret_cast<__bf16 *>(buf);
    __bf16 *lo = hi + kChunk * kLdKt;
    const int off = (16 * rt + (l & 15)) * kLdKt + 32 * ks + 8 * (l >> 4);
    *reinterpret_cast<bf16x8 *>(hi + off) = f.hi;
    *reinterpret_cast<bf16x8 *>(lo + off) = f.lo;
  }
  // Fragment (it, ks) of K^T: row i = 16 it + l % 16, indices (tokens)
  // t = 32 ks + 8 (l / 16) .. +7, as two transpose reads per plane.
  static __device__ __forceinline__ Op<Prec::BF16X3>::Frag get(const uint8_t *buf, int it, int ks) {
    const int l = lane_id(), s = l & 15;
    const __bf16 *hi = reinterpret_cast<const __bf16 *>(buf);
    const __bf16 *lo = hi + kChunk * kLdKt;
    const int off = (32 * ks + 8 * (l >> 4) + (s >> 2)) * kLdKt + 16 * it + 4 * (s & 3);
    const s16x4 h0 = lds_read_tr16(hi + off), h1 = lds_read_tr16(hi + off + 4 * kLdKt);
    const s16x4 l0 = lds_read_tr16(lo + off), l1 = lds_read_tr16(lo + off + 4 * kLdKt);
    Op<Prec::BF16X3>::Frag f;
    f.hi = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
    f.lo = __builtin_bit_cast(bf16x8, __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7));
    return f;
  }
};
// F32 gathers its K^T fragments one value at a time; its row pitch of 132
// floats puts the four lane groups of a gather on two bank halves.
constexpr int kLdKtF32 = kHeadDim + 4;
template <> struct KtLds<Prec::F32> {
  static constexpr int kBytes = kChunk * kLdKtF32 * 4;
  static __device__ __forceinline__ void put(uint8_t *buf, int rt, int ks, const Op<Prec::F32>::Frag &f) {
    const int l = lane_id();
    float *k = reinterpret_cast<float *>(buf) + (16 * rt + (l & 15)) * kLdKtF32 + 32 * ks + 8 * (l >> 4);
    *reinterpret_cast<f32x4 *>(k) = f.a;
    *reinterpret_cast<f32x4 *>(k + 4) = f.b;
  }
  static __device__ __forceinline__ Op<Prec::F32>::Frag get(const uint8_t *buf, int it, int ks) {
    const int l = lane_id();
    const float *k = reinterpret_cast<const float *>(buf) + (32 * ks + 8 * (l >> 4)) * kLdKtF32 + 16 * it + (l & 15);
    Op<Prec::F32>::Frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f.a[e] = k[e * kLdKtF32];
      f.b[e] = k[(e + 4) * kLdKtF32];
    }
    return f;
  }
};

// Fused form: conv + SiLU of 4 raw activations over rows t - 3 .. t.

template <typename Raw>
__device__ __forceinline__ f32x4 conv_silu4(const Raw (&raw)[kConvK], const float4 (&w)[4]) {
  using TA = std::conditional_t<std::is_same<Raw, float4>::value, float, bf16_t>;
  float4 x[kConvK];
#pragma unroll
  for (int r = 0; r < kConvK; ++r) x[r] = RawAct<TA>::f4(raw[r]);
  f32x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    y[e] = siluf_(w[e].x * (&x[0].x)[e] + w[e].y * (&x[1].x)[e] + w[e].z * (&x[2].x)[e] + w[e].w * (&x[3].x)[e]);
  return y;
}

// c[t][d] += a[d] b[t][d] for column tiles t = 0, 1 and contraction steps
// d = 0, 1, each (t, d) into an accumulator of its own. A dependent MFMA
// accumulation waits about 50 cycles for the one before it, while a wave can
// issue an independent MFMA about every 20: BF16X3 therefore issues one split
// pass of all four products at a time, so that no product feeds any of the
// next three.
template <Prec P>
__device__ __forceinline__ void mma_2x2(f32x4 (&c)[2][2], const typename Op<P>::Frag &a0,
                                        const typename Op<P>::Frag &a1, const typename Op<P>::Frag &b00,
                                        const typename Op<P>::Frag &b01, const typename Op<P>::Frag &b10,
                                        const typename Op<P>::Frag &b11) {
  if constexpr (P == Prec::BF16X3) {
    c[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0.hi, b00.hi, c[0][0], 0, 0, 0);
    c[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0.hi, b10.hi, c[1][0], 0, 0, 0);
    c[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1.hi, b01.hi, c[0][1], 0, 0, 0);
    c[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1.hi, b11.hi, c[1][1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);   // keep the passes in this order
    c[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0.hi, b00.lo, c[0][0], 0, 0, 0);
    c[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0.hi, b10.lo, c[1][0], 0, 0, 0);
    c[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1.hi, b01.lo, c[0][1], 0, 0, 0);
    c[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1.hi, b11.lo, c[1][1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    c[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0.lo, b00.hi, c[0][0], 0, 0, 0);
    c[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0.lo, b10.hi, c[1][0], 0, 0, 0);
    c[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1.lo, b01.hi, c[0][1], 0, 0, 0);
    c[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1.lo, b11.hi, c[1][1], 0, 0, 0);
  } else {
    Op<P>::mma2(c[0][0], c[1][0], a0, b00, b10);
    Op<P>::mma2(c[0][1], c[1][1], a1, b01, b11);
  }
}

// ---------------------------------------------------------------------------
// chunk_state: per (sequence, V-head, 32-column slab). 8 waves in two roles
// of four, row tile rt = w % 4: waves 0-3 (x-waves) hold K and Tm rows,
// waves 4-7 (y-waves) Q and P rows. Per chunk c:
//   1. x: X = K S, R = V - diag(Gam) X -> R in LDS      y: Y = Q S
//   2. x: D = Tm R -> D (one buffer per chunk parity) and diag(k~) D in LDS,
//         k~_r = exp(gam_n - gam_r)
//      y: O of chunk c - 1 = s (diag(Gam) Y + P D), from that chunk's D
//   3. all: S <- Gam_n S + K^T diag(k~) D (state rows 16 w) -> S in LDS
// V of chunk c + 1 goes to LDS in step 2 (it is first read in step 1 of that
// chunk). The fused form stages each raw V row of the slab in LDS once and
// the x-waves take conv + SiLU from there, in the time they would otherwise
// wait at the third barrier.
// S lives in two LDS buffers by chunk parity, so that writing the new S
// needs no barrier of its own: three barriers per chunk; the two roles run
// loops of their own (the branch is uniform per wave) with the same
// barriers.
// O trails D by one chunk, so it is formed while the x-waves form D, off the
// chain S -> X -> D -> S that orders the chunks; the last chunk's O follows
// the loop.
// Each role keeps its left operands in registers of its own (K or Q rows: 4
// fragments; Tm or P rows: 2), reloaded for the next chunk right after their
// last use so that the loads overlap the rest of the chunk. No register is
// loaded by both roles, so the compiler's memory-wait counts never make a
// wave wait for loads only the other role issues. The loads that must land
// before a chunk ends (V rows, gam) belong to the x-waves, whose memory
// operations are loads only (checkpoint stores aside), so the y-waves'
// pending O stores never hold them up. The K^T fragments of the state update
// are not loaded: the x-waves leave their K fragments in LDS and every wave
// reads its K^T fragments from there.
// LDS of a chunk_state block, carved from one byte array (16-byte aligned
// parts):
//   Stb: S, the B operand of K S and Q S, by chunk parity
//   Rtb: R, the B operand of Tm R (2 x 2 blocks)
//   Dtb: D, the B operand of P D, by chunk parity
//   Dsb: diag(k~) D, the B operand of K^T (.)
//   Vs:  V rows of the slab (fp32); Os: O staging, 16 rows per y-wave
//   Ktb: K rows of the chunk (for the K^T fragments)
//   Vw:  fused form, conv taps of the slab's V channels
//   Vr:  fused form, raw V rows of the slab by chunk parity (rows 0 .. 2 are
//        the three rows before the chunk, rows 3 .. 66 the chunk's own)
//   G_s: exp(gam_r); Ksc: exp(gam_n - gam_r)
template <Prec P, typename TA, bool kFused> struct StateLds {
  static constexpr int kVrRows = kFused ? kChunk + kConvK - 1 : 1;
  static constexpr size_t kStb = 0;
  static constexpr size_t kRtb = kStb + 2 * 8 * kLdsBlk;
  static constexpr size_t kDtb = kRtb + 4 * kLdsBlk;
  static constexpr size_t kDsb = kDtb + 2 * 4 * kLdsBlk;
  static constexpr size_t kVs = kDsb + 4 * kLdsBlk;
  static constexpr size_t kOs = kVs + kChunk * kLdV * sizeof(float);
  static constexpr size_t kKtb = kOs + 4 * 16 * kLdOs * sizeof(float);
  static constexpr size_t kVw = kKtb + (KtLds<P>::kBytes + 15) / 16 * 16;
  static constexpr size_t kVr = kVw + (kFused ? kSlab : 1) * sizeof(float4);
  static constexpr size_t kG = kVr + ((kFused ? 2 : 1) * kVrRows * kSlab * sizeof(TA) + 15) / 16 * 16;
  static constexpr size_t kKsc = kG + kChunk * sizeof(float);
  static constexpr size_t kBytes = kKsc + kChunk * sizeof(float);
};

template <Prec P, typename TA, bool kFused, bool kCkpt>
__global__ __launch_bounds__(kStateThreads) void chunk_state_kernel(PrefillParams p, int64_t max_chunks) {
  using Frag = typename Op<P>::Frag;
  using SL = StateLds<P, TA, kFused>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SL::kBytes];
  uint8_t (*Stb)[8 * kLdsBlk] = reinterpret_cast<uint8_t (*)[8 * kLdsBlk]>(smem + SL::kStb);
  uint8_t *Rtb = smem + SL::kRtb;
  uint8_t (*Dtb)[4 * kLdsBlk] = reinterpret_cast<uint8_t (*)[4 * kLdsBlk]>(smem + SL::kDtb);
  uint8_t *Dsb = smem + SL::kDsb;
  float *Vs = reinterpret_cast<float *>(smem + SL::kVs);
  float *Os = reinterpret_cast<float *>(smem + SL::kOs);
  uint8_t *Ktb = smem + SL::kKtb;
  float4 *Vw = reinterpret_cast<float4 *>(smem + SL::kVw);
  TA (*Vr)[SL::kVrRows][kSlab] = reinterpret_cast<TA (*)[SL::kVrRows][kSlab]>(smem + SL::kVr);
  float *G_s = reinterpret_cast<float *>(smem + SL::kG);
  float *ksc_s = reinterpret_cast<float *>(smem + SL::kKsc);

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();
  const int rt = __builtin_amdgcn_readfirstlane(wave) & 3;        // uniform per wave
  const bool x_wave = __builtin_amdgcn_readfirstlane(wave) < 4;
  const int lr = 4 * (lane >> 4);    // accumulator row offset of this lane
  const int lc = lane & 15;          // accumulator column of this lane
  // Block order: workgroups are dealt to the 8 XCDs round-robin (block b on
  // XCD b % 8), each with its own L2. Blocks b = 32 g + 8 s + x hold slab s
  // of (sequence, V-head) pair 8 g + x, so the 4 slabs of a pair, and the
  // V-heads j, j + 8, ... that share K-head operands, run on one XCD and
  // share its L2.
  if constexpr (kFused) {
    const int first_fold = static_cast<int>(gridDim.x) - p.fold_blocks;
    if (p.fold_blocks > 0 && static_cast<int>(blockIdx.x) >= first_fold) {
      fold_norm<TA>(p, max_chunks, blockIdx.x - first_fold);
      return;
    }
  }
  const int nslab = kHeadDim / kSlab;
  const int pair = kXcds * (blockIdx.x / (kXcds * nslab)) + blockIdx.x % kXcds;
  const int slab = (blockIdx.x / kXcds) % nslab;
  if (pair >= p.n_seqs * p.n_v) return;
  const int j = pair % p.n_v;
  const int n = pair / p.n_v;
  const int hk = j % p.n_qk;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  if (seq0 < 0 || L < 0 || seq0 + L > p.n_tokens) return;
  const int nchunks = (L + kChunk - 1) / kChunk;
  const int cid0 = first_unit(p.cu, n, kChunk, 0);
  // Chunk ids past the workspace only arise from cu_seqlens outside the
  // contract; never index past the workspace.
  if (cid0 + nchunks > max_chunks) return;
  const Workspace ws = carve(p.ws, max_chunks, p.n_qk, p.n_v);
  const float scale = 0.08838834764831845f;  // 1/sqrt(128)
  const int col_base = slab * kSlab;
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
  for (int ct = 0; ct < 2; ++ct) lds_put4<P>(Stb[0], 4, 16 * wave + lr, 16 * ct + lc, S[ct]);

  // Operand sources of chunk c (fragment-major blocks).
  const size_t qk_step = static_cast<size_t>(p.n_qk) * kQkBytes;
  const size_t v_step = static_cast<size_t>(p.n_v) * kVBytes;
  const uint8_t *k_src0 = ws.qk + (static_cast<size_t>(cid0) * p.n_qk + hk) * kQkBytes;   // K rows
  const uint8_t *q_src0 = k_src0 + kKBytes;                                               // Q rows
  const uint8_t *t_src0 = ws.v + (static_cast<size_t>(cid0) * p.n_v + j) * kVBytes;       // Tm rows
  const uint8_t *p_src0 = t_src0 + kMatBytes;                                             // P rows
  // V rows (x-waves): thread tid holds row tid / 4, slab channels
  // 8 (tid % 4) .. +7.
  const int v_row = (tid & (4 * kWave - 1)) >> 2, v_c8 = tid & 3;

  Frag fk[kHeadDim / 32], fq[kHeadDim / 32], ft[kChunk / 32], fp[kChunk / 32];
  f32x4 pv[2];
  // Fused form: the raw row of this thread's 8 V channels is loaded once per
  // chunk (16 bytes for bf16, 32 for fp32), with the other operands of the
  // next chunk, and staged in Vr, where every thread reads the four rows its
  // conv needs.
  using Raw = typename RawAct<TA>::type;
  constexpr int kRawQ = static_cast<int>(sizeof(TA)) / 2;   // 16-byte pieces per 8 channels
  uint4 vr[kRawQ];
  const int Cq = kHeadDim * (2 * p.n_qk + p.n_v);
  const int vch0 = 2 * p.n_qk * kHeadDim + j * kHeadDim + col_base;   // first slab channel in qkv
  constexpr int kHalo = kConvK - 1;
  if constexpr (kFused) {
    if (tid < kSlab) Vw[tid] = reinterpret_cast<const float4 *>(p.conv_w)[vch0 + tid];
    // Chunk 0's raw rows and the conv state before it; rows 61 .. 63 also
    // seed the next chunk's first three rows.
    if (nchunks > 0 && x_wave) {
      const int row = min(v_row, min(kChunk, L) - 1);
      const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const TA *>(p.qkv) +
                                                         static_cast<size_t>(seq0 + row) * Cq + vch0 + 8 * v_c8);
      uint4 *dst = reinterpret_cast<uint4 *>(&Vr[0][kHalo + v_row][8 * v_c8]);
#pragma unroll
      for (int q = 0; q < kRawQ; ++q) dst[q] = src[q];
      if (v_row >= kChunk - kHalo) {
        uint4 *dn = reinterpret_cast<uint4 *>(&Vr[1][v_row - (kChunk - kHalo)][8 * v_c8]);
#pragma unroll
        for (int q = 0; q < kRawQ; ++q) dn[q] = src[q];
      }
      if (tid < kHalo * 4) {
        const int hr = tid >> 2, hc = tid & 3;
        const uint4 *hs = reinterpret_cast<const uint4 *>(static_cast<const TA *>(p.st_in) +
                                                          (static_cast<size_t>(n) * kHalo + hr) * Cq + vch0 + 8 * hc);
        uint4 *hd = reinterpret_cast<uint4 *>(&Vr[0][hr][8 * hc]);
#pragma unroll
        for (int q = 0; q < kRawQ; ++q) hd[q] = hs[q];
      }
    }
    block_sync_lds();
  }
  double pg = 0.0, pg_end = 0.0;

#define GDN_LOAD_ROWS(dst, src0, c)                                                                   \
  _Pragma("unroll") for (int ks = 0; ks < kHeadDim / 32; ++ks)                                       \
    dst[ks] = FragIO<P>::load(src0 + (c) * qk_step, kHeadDim / 32, rt, ks)
  // Row tiles 0 and 1 of Tm and P end before column 32: their second k
  // step is zero and skipped.
#define GDN_LOAD_MAT(dst, src0, c)                                                                    \
  _Pragma("unroll") for (int ks = 0; ks < kChunk / 32; ++ks)                                         \
    if (ks == 0 || rt >= 2) dst[ks] = FragIO<P>::load(src0 + (c) * v_step, kChunk / 32, rt, ks)
  // V slab rows and gam of chunk c (x-waves; committed to LDS after the chunk
  // before it).
#define GDN_LOAD_VG(c)                                                                               \
  do {                                                                                               \
    const int t0_ = seq0 + (c) * kChunk, len_ = min(kChunk, L - (c) * kChunk);                       \
    if constexpr (kFused) {                                                                          \
      const uint4 *src_ = reinterpret_cast<const uint4 *>(static_cast<const TA *>(p.qkv) +           \
                                                          static_cast<size_t>(t0_ + min(v_row, len_ - 1)) * Cq + \
                                                          vch0 + 8 * v_c8);                          \
      _Pragma("unroll") for (int q_ = 0; q_ < kRawQ; ++q_) vr[q_] = src_[q_];                        \
    } else {                                                                                         \
      const float *src_ = p.v + (t0_ + min(v_row, len_ - 1)) * v_stride + j * kHeadDim + col_base + 8 * v_c8; \
      pv[0] = *reinterpret_cast<const f32x4 *>(src_);                                                \
      pv[1] = *reinterpret_cast<const f32x4 *>(src_ + 4);                                            \
    }                                                                                                \
    if (tid < kChunk) {                                                                              \
      const double *gm = ws.gam + (static_cast<size_t>(cid0 + (c)) * p.n_v + j) * kChunk;            \
      pg = gm[tid];                                                                                  \
      pg_end = gm[kChunk - 1];                                                                       \
    }                                                                                                \
  } while (0)
  // Fused form: the raw row of chunk c to Vr (rows 61 .. 63 also to the
  // other buffer, as the first rows of chunk c + 1); visible after the next
  // barrier.
#define GDN_STAGE_V(c)                                                                               \
  do {                                                                                               \
    if constexpr (kFused) {                                                                          \
      uint4 *dst_ = reinterpret_cast<uint4 *>(&Vr[(c) & 1][kHalo + v_row][8 * v_c8]);                \
      _Pragma("unroll") for (int q_ = 0; q_ < kRawQ; ++q_) dst_[q_] = vr[q_];                        \
      if (v_row >= kChunk - kHalo) {                                                                 \
        uint4 *dn_ = reinterpret_cast<uint4 *>(&Vr[((c) + 1) & 1][v_row - (kChunk - kHalo)][8 * v_c8]); \
        _Pragma("unroll") for (int q_ = 0; q_ < kRawQ; ++q_) dn_[q_] = vr[q_];                       \
      }                                                                                              \
    }                                                                                                \
  } while (0)
  // V rows of chunk c to LDS, formed after the chunk's second barrier (the
  // previous chunk's V has been read by then) and before its third, while
  // the waves would otherwise wait (it is off the chain). Rows past the
  // chunk's length were loaded from its last row and are zeroed here, at
  // first use, so that the loads stay in flight until then.
  // Fused form: conv + SiLU of the staged raw rows (rows t - 3 .. t of row t
  // sit at Vr rows t .. t + 3) of the thread's channels 8 (tid % 4) + 4 h
  // .. +3, both halves on the x-waves: the y-waves, which form O in the same
  // interval, arrive at the third barrier later.
#define GDN_FORM_V(c, h)                                                                             \
  do {                                                                                               \
    Raw raw_[kConvK];                                                                                \
    _Pragma("unroll") for (int k_ = 0; k_ < kConvK; ++k_)                                            \
      raw_[k_] = *reinterpret_cast<const Raw *>(&Vr[(c) & 1][v_row + k_][8 * v_c8 + 4 * (h)]);        \
    const float4 w_[4] = {Vw[8 * v_c8 + 4 * (h)], Vw[8 * v_c8 + 4 * (h) + 1], Vw[8 * v_c8 + 4 * (h) + 2], \
                          Vw[8 * v_c8 + 4 * (h) + 3]};                                               \
    const f32x4 y_ = conv_silu4(raw_, w_);                                                           \
    const f32x4 zv_ = {0.f, 0.f, 0.f, 0.f};                                                          \
    *reinterpret_cast<f32x4 *>(Vs + v_row * kLdV + 8 * v_c8 + 4 * (h)) =                             \
        v_row < min(kChunk, L - (c) * kChunk) ? y_ : zv_;                                            \
  } while (0)
  // Unfused form: the loaded V rows (x-waves).
#define GDN_WRITE_V(c)                                                                               \
  do {                                                                                               \
    const int lenv_ = min(kChunk, L - (c) * kChunk);                                                 \
    const f32x4 zv_ = {0.f, 0.f, 0.f, 0.f};                                                          \
    float *dst_ = Vs + v_row * kLdV + 8 * v_c8;                                                      \
    *reinterpret_cast<f32x4 *>(dst_) = v_row < lenv_ ? pv[0] : zv_;                                  \
    *reinterpret_cast<f32x4 *>(dst_ + 4) = v_row < lenv_ ? pv[1] : zv_;                              \
  } while (0)
  // gam of chunk c to LDS (after the chunk's last barrier: the y-waves read
  // the previous chunk's decays up to it).
#define GDN_COMMIT_G()                                                                               \
  do {                                                                                               \
    if (tid < kChunk) {                                                                              \
      G_s[tid] = expf(static_cast<float>(pg));                                                       \
      ksc_s[tid] = expf(static_cast<float>(pg_end - pg));                                            \
    }                                                                                                \
  } while (0)

  // y-waves: O rows 16 rt of chunk c = s * acc, staged in LDS and written out
  // with one 16-byte store per lane (bf16) or two (fp32).
  auto store_o = [&](int c, const f32x4 (&acc)[2]) {
    const int t0_ = seq0 + c * kChunk, len_ = min(kChunk, L - c * kChunk);
    float *Ow = Os + rt * 16 * kLdOs;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) Ow[acc_row(r) * kLdOs + 16 * ct + acc_col()] = scale * acc[ct][r];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave reads back only its own rows
    const int orow = lane >> 2, oc = 8 * (lane & 3);
    const float *src = Ow + orow * kLdOs + oc;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(src);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(src + 4);
    if (16 * rt + orow < len_) {
      const size_t dst = (t0_ + 16 * rt + orow) * v_stride + j * kHeadDim + col_base + oc;
      if (kFused && p.fold_blocks > 0) {
        fold_put4(o, dst, a);
        fold_put4(o, dst + 4, b);
      } else {
        Act<TA>::store4(o, dst, make_float4(a[0], a[1], a[2], a[3]));
        Act<TA>::store4(o, dst + 4, make_float4(b[0], b[1], b[2], b[3]));
      }
    }
  };
  // Folded norm: this y-wave's o rows of chunk c are stored; count them in.
  auto publish = [&](int c) {
    if constexpr (kFused) {
      if (p.fold_blocks > 0) {
        uint32_t *ctr = p.ready + (static_cast<size_t>(cid0 + c) * p.n_v + j) * kReadyStride;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the o stores have completed
        if (lane == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };

  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // out[t] = a S over rows 16 rt, column tile t: all eight S fragments are
  // read first, then the products run as four accumulation chains.
  auto times_s = [&](const Frag (&a)[kHeadDim / 32], const uint8_t *sbuf, f32x4 (&out)[2]) {
    Frag b[2][kHeadDim / 32];
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 32; ++ks) {
      b[0][ks] = lds_frag<P>(sbuf, ks);
      b[1][ks] = lds_frag<P>(sbuf, kHeadDim / 32 + ks);
    }
    __builtin_amdgcn_sched_barrier(0);       // every read in flight before the first product
    f32x4 c[2][2] = {{zero4, zero4}, {zero4, zero4}};
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 32; ks += 2)
      mma_2x2<P>(c, a[ks], a[ks + 1], b[0][ks], b[0][ks + 1], b[1][ks], b[1][ks + 1]);
    out[0] = c[0][0] + c[0][1];
    out[1] = c[1][0] + c[1][1];
  };
  // out[t] += a B over rows 16 rt for a 64 x 32 right operand B in LDS (R or
  // D); row tiles 0 and 1 of the lower-triangular a end before column 32.
  auto times_mat = [&](const Frag (&a)[kChunk / 32], const uint8_t *buf, f32x4 (&out)[2]) {
    const Frag b00 = lds_frag<P>(buf, 0), b10 = lds_frag<P>(buf, 2);
    if (rt >= 2) {
      const Frag b01 = lds_frag<P>(buf, 1), b11 = lds_frag<P>(buf, 3);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 c[2][2] = {{out[0], zero4}, {out[1], zero4}};
      mma_2x2<P>(c, a[0], a[1], b00, b01, b10, b11);
      out[0] = c[0][0] + c[0][1];
      out[1] = c[1][0] + c[1][1];
    } else {
      Op<P>::mma2(out[0], out[1], a[0], b00, b10);
    }
  };

  // 3. S <- Gam_n S + K^T (diag(k~) D), state rows 16 wave; then the
  // checkpoint (the state after token (ci + 1) * 64 of the sequence) and S
  // to the other S buffer, whose last readers (chunk ci - 1) are done.
  auto update_state = [&](int ci, float g_end) {
    block_sync_lds();                        // D and diag(k~) D visible
    {
      const Frag k0 = KtLds<P>::get(Ktb, wave, 0), k1 = KtLds<P>::get(Ktb, wave, 1);
      const Frag d00 = lds_frag<P>(Dsb, 0), d01 = lds_frag<P>(Dsb, 1);
      const Frag d10 = lds_frag<P>(Dsb, 2), d11 = lds_frag<P>(Dsb, 3);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 c[2][2] = {{S[0] * g_end, zero4}, {S[1] * g_end, zero4}};
      mma_2x2<P>(c, k0, k1, d00, d01, d10, d11);
      S[0] = c[0][0] + c[0][1];
      S[1] = c[1][0] + c[1][1];
    }
    if constexpr (kCkpt) {
      if ((ci + 1) % p.ckpt_chunks == 0 && (ci + 1) * kChunk <= L) {
        const int c = (ci + 1) / p.ckpt_chunks - 1;
        if (c < p.ckpt_cap) {
          float *dst = p.S_ckpt + ((static_cast<size_t>(n) * p.ckpt_cap + c) * p.n_v + j) * kHeadDim * kHeadDim;
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              dst[static_cast<size_t>(16 * wave + acc_row(r)) * kHeadDim + col_base + 16 * ct + acc_col()] = S[ct][r];
        }
      }
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) lds_put4<P>(Stb[(ci + 1) & 1], 4, 16 * wave + lr, 16 * ct + lc, S[ct]);
  };

  // The two roles run loops of their own (the branch is uniform per wave),
  // with the same three barriers per chunk.
  if (x_wave) {
    if (nchunks > 0) {
      GDN_LOAD_ROWS(fk, k_src0, 0);
      GDN_LOAD_MAT(ft, t_src0, 0);
      GDN_LOAD_VG(0);
      if constexpr (kFused) { GDN_FORM_V(0, 0); GDN_FORM_V(0, 1); }
      else GDN_WRITE_V(0);
      GDN_COMMIT_G();
    }
    for (int ci = 0; ci < nchunks; ++ci) {
      // Operands of the next chunk (the last chunk reloads itself, so every
      // iteration issues the same loads).
      const int cn = min(ci + 1, nchunks - 1);
      block_sync_lds();                      // S, V, gam of chunk ci visible
      const float g_end = G_s[kChunk - 1];
      GDN_LOAD_VG(cn);
      // 1. X = K S, rows 16 rt, both column tiles; R = V - diag(Gam) X.
      f32x4 X[2];
      times_s(fk, Stb[ci & 1], X);
#pragma unroll
      for (int ks = 0; ks < kHeadDim / 32; ++ks) KtLds<P>::put(Ktb, rt, ks, fk[ks]);
      GDN_LOAD_ROWS(fk, k_src0, cn);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f32x4 rv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * rt + acc_row(r);
          rv[r] = Vs[row * kLdV + 16 * ct + acc_col()] - G_s[row] * X[ct][r];
        }
        lds_put4<P>(Rtb, 2, 16 * rt + lr, 16 * ct + lc, rv);
      }
      GDN_STAGE_V(cn);
      block_sync_lds();                      // R (and the raw V rows) visible
      // 2. D = Tm R, rows 16 rt -> D and diag(k~) D in LDS.
      f32x4 acc[2] = {zero4, zero4};
      times_mat(ft, Rtb, acc);
      GDN_LOAD_MAT(ft, t_src0, cn);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        lds_put4<P>(Dtb[ci & 1], 2, 16 * rt + lr, 16 * ct + lc, acc[ct]);
        f32x4 ds;
#pragma unroll
        for (int r = 0; r < 4; ++r) ds[r] = acc[ct][r] * ksc_s[16 * rt + acc_row(r)];
        lds_put4<P>(Dsb, 2, 16 * rt + lr, 16 * ct + lc, ds);
      }
      if constexpr (kFused) { GDN_FORM_V(cn, 0); GDN_FORM_V(cn, 1); }
      else GDN_WRITE_V(cn);
      update_state(ci, g_end);
      GDN_COMMIT_G();
    }
  } else {
    f32x4 oy[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};   // diag(Gam) Y of the previous chunk
    if (nchunks > 0) {
      GDN_LOAD_ROWS(fq, q_src0, 0);
      GDN_LOAD_MAT(fp, p_src0, 0);
    }
    for (int ci = 0; ci < nchunks; ++ci) {
      const int cn = min(ci + 1, nchunks - 1);
      block_sync_lds();                      // S, V, gam of chunk ci visible
      // Chunk ci - 2's o rows went out in the last iteration, and this
      // wave's loads of then are needed now: counting them in waits for
      // nothing else.
      if (ci >= 2) publish(ci - 2);
      const float g_end = G_s[kChunk - 1];
      // 1. Y = Q S, rows 16 rt, both column tiles.
      f32x4 Y[2];
      times_s(fq, Stb[ci & 1], Y);
      GDN_LOAD_ROWS(fq, q_src0, cn);
      block_sync_lds();                      // (the x-waves' R)
      // 2. O of the previous chunk = s (diag(Gam) Y + P D).
      if (ci > 0) {
        f32x4 acc[2] = {oy[0], oy[1]};
        times_mat(fp, Dtb[(ci - 1) & 1], acc);
        GDN_LOAD_MAT(fp, p_src0, ci);
        store_o(ci - 1, acc);
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) oy[ct][r] = G_s[16 * rt + acc_row(r)] * Y[ct][r];
      update_state(ci, g_end);
    }
    // O of the last chunk (its D was made visible by the loop's barriers).
    if (nchunks > 0) {
      const int cl = nchunks - 1;
      if (cl >= 1) publish(cl - 1);
      f32x4 acc[2] = {oy[0], oy[1]};
      times_mat(fp, Dtb[cl & 1], acc);
      store_o(cl, acc);
      publish(cl);
    }
  }
#undef GDN_LOAD_ROWS
#undef GDN_LOAD_MAT
#undef GDN_LOAD_VG
#undef GDN_STAGE_V
#undef GDN_FORM_V
#undef GDN_WRITE_V
#undef GDN_COMMIT_G

#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      p.S_out[sbase + static_cast<size_t>(16 * wave + acc_row(r)) * kHeadDim + col_base + 16 * ct + acc_col()] = S[ct][r];
}

}  // namespace

int prefill_fold_blocks(int n_seqs, int n_v) {
  constexpr int64_t kCUs = 256, kMinFold = 32, kMaxFold = 64;
  const int64_t pairs = static_cast<int64_t>(n_seqs) * n_v;
  const int64_t slab_blocks = (pairs + kXcds - 1) / kXcds * kXcds * (kHeadDim / kSlab);
  const int64_t idle = kCUs - slab_blocks;
  return idle >= kMinFold ? static_cast<int>(idle < kMaxFold ? idle : kMaxFold) : 0;
}

size_t prefill_workspace_bytes(int n_seqs, int n_tokens, int n_qk, int n_v) {
  const int64_t chunks = max_chunks(n_seqs, n_tokens);
  return static_cast<size_t>(chunks) * (n_qk * kQkBytes + n_v * (kVBytes + kChunk * sizeof(double)));
}

hipError_t launch_prefill(const PrefillParams &p, gdn_dtype act, hipStream_t s) {
  const int64_t chunks = max_chunks(p.n_seqs, p.n_tokens);
  const dim3 grid_local(static_cast<unsigned>(chunks), static_cast<unsigned>(p.n_qk));
  const int64_t pairs = static_cast<int64_t>(p.n_seqs) * p.n_v;
  const dim3 grid_state(static_cast<unsigned>((pairs + kXcds - 1) / kXcds * kXcds * (kHeadDim / kSlab) +
                                             (p.qkv != nullptr ? p.fold_blocks : 0)));
  const bool fused = p.qkv != nullptr;
#define GDN_LAUNCH(PR, TA, FU)                                                                                \
  do {                                                                                                        \
    if (p.n_tokens > 0)                                                                                       \
      hipLaunchKernelGGL((chunk_local_kernel<PR, TA, FU>), grid_local, dim3(kLocalThreads), 0, s, p, chunks); \
    if (p.ckpt_chunks > 0)                                                                                    \
      hipLaunchKernelGGL((chunk_state_kernel<PR, TA, FU, true>), grid_state, dim3(kStateThreads), 0, s, p,     \
                         chunks);                                                                             \
    else                                                                                                      \
      hipLaunchKernelGGL((chunk_state_kernel<PR, TA, FU, false>), grid_state, dim3(kStateThreads), 0, s, p,    \
                         chunks);                                                                             \
  } while (0)
  if (act == GDN_BF16) {
    if (fused) GDN_LAUNCH(Prec::BF16X3, bf16_t, true);
    else GDN_LAUNCH(Prec::BF16X3, bf16_t, false);
  } else {
    if (fused) GDN_LAUNCH(Prec::F32, float, true);
    else GDN_LAUNCH(Prec::F32, float, false);
  }
#undef GDN_LAUNCH
  return hipGetLastError();
}

}  // namespace gdn
