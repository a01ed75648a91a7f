// gemm.hip -- the bf16 products around the mixer: the input projections
// (attn_qkv, attn_gate, ssm_beta, ssm_alpha of the layer input) and ssm_out
// (the xwen CLAUDE.md page, section "Architecture cheat sheet", gated DeltaNet
// paragraph).
//
//   out[m][n] = sum_k x[m][k] * w[n][k]      x [M][K], w [N][K] (Linear layout)
//
// bf16 operands, fp32 accumulation, each output rounded once to bf16. The N
// output columns are split into up to 4 segments: segment s covers columns
// [start[s], start[s+1]), reads its weight rows from w[s] and writes out[s]
// with row pitch ld[s], so the four input projections run as one product
// without stacking their weights.
//
// Tiling for gfx950. A block of 8 waves owns a kBM x BN tile (BN = 32 * WN):
// waves 0-3 only compute, waves 4-7 only issue the operand loads, so that a
// load instruction never holds up the issue of a compute wave's MFMAs (a
// vector-memory instruction stalls the wave that issues it). Compute wave
// (wr, wc) owns rows 128 wr .. +127 and columns 16 WN wc .. +16 WN - 1,
// i.e. 8 x WN accumulator tiles of 16 x 16 (v_mfma_f32_16x16x32_bf16). The
// contraction runs in k-tiles of 64 staged in an LDS ring (3 deep; 4 for the
// decode-sized tiles; see gemm_dma_kernel), one barrier per k-tile. An LDS row is the 128 bytes of
// one operand row in a k-tile, as 8 chunks of 16 bytes (8 k values); chunk c
// of row r is stored at slot c ^ (r & 7), which makes both the 16-byte writes
// and the 16-byte fragment reads free of bank conflicts.
//
// 17 to 64 rows (decode batches) take the same kernel with tiles of 32 or 64
// rows (launch_decode); up to 16 rows take gemm_skinny_kernel instead, which
// streams the weights once and splits the work over the contraction.
//
// The weight fragment is the MFMA's first operand and the activation fragment
// its second, so an accumulator lane holds 4 consecutive output columns of
// one row: stores are 8 bytes per lane.
//
// Tile order: blocks are dealt round-robin to the 8 XCDs; each XCD takes a
// contiguous range of tiles, walked in groups of kGroupM row tiles so that
// the blocks running together on one XCD share operand panels in its L2.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kBM = 256;          // rows of a block tile (2 waves x 8 fragments x 16)
constexpr int kBK = 64;           // contraction indices per k-tile
constexpr int kRowBytes = kBK * 2;
constexpr int kGemmThreads = 512;          // 4 compute waves + 4 load waves
constexpr int kComputeThreads = 256;
constexpr int kGroupM = 4;        // row tiles per group in the tile walk
constexpr int kGemmXcds = 8;
// Per-lane source addresses of the 8 loads of a k-tile. A vector value, not
// an array: the compiler may move a private array into LDS or scratch.
typedef uint64_t u64x8 __attribute__((ext_vector_type(8)));

template <typename T>
__device__ __forceinline__ T sel4(int s, T a0, T a1, T a2, T a3) {
  return s == 0 ? a0 : s == 1 ? a1 : s == 2 ? a2 : a3;
}

// The segment table, read once into scalars. Indexing the kernel argument's
// arrays with a runtime segment number would make the compiler copy the whole
// argument to private memory (or LDS) first.
struct Segs {
  int n_seg, N, s1, s2, s3;
  const uint16_t *w0, *w1, *w2, *w3;
  uint16_t *o0, *o1, *o2, *o3;
  int64_t l0, l1, l2, l3;

  __device__ __forceinline__ explicit Segs(const GemmParams &p)
      : n_seg(p.n_seg), N(p.N), s1(p.start[1]), s2(p.start[2]), s3(p.start[3]),
        w0(p.w[0]), w1(p.w[1]), w2(p.w[2]), w3(p.w[3]), o0(p.out[0]), o1(p.out[1]), o2(p.out[2]),
        o3(p.out[3]), l0(p.ld[0]), l1(p.ld[1]), l2(p.ld[2]), l3(p.ld[3]) {}
  // Segment of column n.
  __device__ __forceinline__ int seg(int n) const {
    return (n_seg > 1 && n >= s1) + (n_seg > 2 && n >= s2) + (n_seg > 3 && n >= s3);
  }
  __device__ __forceinline__ int start(int s) const { return sel4(s, 0, s1, s2, s3); }
  __device__ __forceinline__ int end(int s) const { return s + 1 < n_seg ? sel4(s, s1, s2, s3, N) : N; }
  __device__ __forceinline__ const uint16_t *w(int s) const { return sel4(s, w0, w1, w2, w3); }
  __device__ __forceinline__ uint16_t *out(int s) const { return sel4(s, o0, o1, o2, o3); }
  __device__ __forceinline__ int64_t ld(int s) const { return sel4(s, l0, l1, l2, l3); }
};

// Byte offset of chunk c of LDS row r.
__device__ __forceinline__ int lds_off(int r, int c) { return r * kRowBytes + ((c ^ (r & 7)) << 4); }

// Epilogue: acc[i][j] of this lane holds out[mrow + 16 i][ncol + 16 j + e],
// e = 0..3 (4 consecutive columns: one 8-byte store when they stay in one
// segment and are aligned, else one 2-byte store each).
// Four columns n .. n+3 of row m that cross a segment end, the last column or
// an 8-byte boundary: one 2-byte store each. Kept out of line so that the
// epilogue loop stays small enough to unroll (the accumulators then stay in
// registers).
__device__ __noinline__ void store4_split(Segs g, int m, int n, uint32_t lo, uint32_t hi) {
  for (int e = 0; e < 4; ++e) {
    const int ne = n + e;
    if (ne < g.N) {
      const int se = g.seg(ne);
      const uint16_t h = static_cast<uint16_t>(((e < 2 ? lo : hi) >> (16 * (e & 1))) & 0xffff);
      g.out(se)[static_cast<int64_t>(m) * g.ld(se) + (ne - g.start(se))] = h;
    }
  }
}

template <int TM, int WN>
__device__ __forceinline__ void gemm_epilogue(const Segs &g, int M, const f32x4 (&acc)[TM][WN], int mrow, int ncol) {
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int m = mrow + 16 * i, n = ncol + 16 * j;
      const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(acc[i][j][0])) |
                          (static_cast<uint32_t>(f32_to_bf16(acc[i][j][1])) << 16);
      const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(acc[i][j][2])) |
                          (static_cast<uint32_t>(f32_to_bf16(acc[i][j][3])) << 16);
      if (m < M && n < g.N) {
        const int s = g.seg(n);
        uint16_t *dst = g.out(s) + static_cast<int64_t>(m) * g.ld(s) + (n - g.start(s));
        if (n + 4 <= g.end(s) && (reinterpret_cast<uintptr_t>(dst) & 7) == 0)
          *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
        else
          store4_split(g, m, n, lo, hi);
      }
    }
  }
}

// The operand tiles are brought into LDS by the load instructions
// themselves (16 bytes per lane, written at the wave's LDS address +
// 16 * lane), in a ring of kStages k-tiles: the loads of k-tile kt + 2 are
// issued as soon as every wave has finished k-tile kt - 1, so two k-tiles of
// memory latency hide behind the MFMAs, and no registers stage the data. Each
// lane loads the chunk that belongs in its slot of the swizzled row: chunk
// (lane & 7) ^ (row & 7).
constexpr int kStages = 3;
constexpr int kMaxWn = 5;         // kStages k-tiles of 256 + 32 WN rows fit the 160 KB of LDS

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  // This wave's loads except the newest N have landed in LDS, its LDS reads
  // are done; then the workgroup barrier (which waits for nothing else, so
  // the newest k-tile stays in flight).
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// The same with the newest `newer` k-tiles of L loads each still in flight
// (newer <= S - 2).
template <int L, int S>
__device__ __forceinline__ void wait_vm_barrier_tiles(int newer) {
#define GDN_WAIT_CASE(c) \
  if constexpr ((c) <= S - 2) { if (newer == (c)) { wait_vm_barrier<L * (c)>(); return; } }
  GDN_WAIT_CASE(7) GDN_WAIT_CASE(6) GDN_WAIT_CASE(5) GDN_WAIT_CASE(4)
  GDN_WAIT_CASE(3) GDN_WAIT_CASE(2) GDN_WAIT_CASE(1)
#undef GDN_WAIT_CASE
  wait_vm_barrier<0>();
}

// One block tile of 32 TM rows x 32 WN columns at (m0, n0): compute wave
// (wr, wc) owns rows 16 TM wr .. +16 TM - 1, i.e. TM x WN accumulator tiles.
// smem holds a ring of S k-tiles of this shape, S - 1 of them loaded ahead.
template <int TM, int WN, int S = kStages>
__device__ __forceinline__ void gemm_tile(const GemmParams &p, uint8_t *smem, int m0, int n0) {
  constexpr int BM = 32 * TM, BN = 32 * WN;
  constexpr int kAChunks = BM * 8 / kComputeThreads;
  constexpr int kBChunks = BN * 8 / kComputeThreads;
  constexpr int kLoads = kAChunks + kBChunks;     // loads per thread and k-tile
  constexpr int kABytes = BM * kRowBytes, kBBytes = BN * kRowBytes, kStage = kABytes + kBBytes;
  static_assert(kAChunks <= 8 && kBChunks <= 8, "at most 8 chunks per operand and thread");

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform per wave
  const bool loader = wave >= 4;
  const int wr = (wave & 3) >> 1, wc = wave & 1;
  const int K = p.K;
  const Segs g(p);

  // Load waves: load i of this lane is row lrow + 32 i of the tile, the
  // chunk for slot lane & 7.
  const int ltid = tid & (kComputeThreads - 1);
  const int lrow = ltid >> 3;
  const int gchunk = (lane & 7) ^ (lrow & 7);
  u64x8 asrc = {}, bsrc = {};
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    const int m = min(m0 + lrow + 32 * i, p.M - 1);
    asrc[i] = reinterpret_cast<uint64_t>(p.x + static_cast<int64_t>(m) * K + 8 * gchunk);
  }
#pragma unroll
  for (int i = 0; i < kBChunks; ++i) {
    const int n = min(n0 + lrow + 32 * i, p.N - 1);
    const int s = g.seg(n);
    bsrc[i] = reinterpret_cast<uint64_t>(g.w(s) + static_cast<int64_t>(n - g.start(s)) * K + 8 * gchunk);
  }
  const int wdst = 8 * (wave & 3) * kRowBytes;    // this wave's 8 rows of load i: + 32 i rows

#define GDN_REP8(M) M(0) M(1) M(2) M(3) M(4) M(5) M(6) M(7)
#define GDN_DMA(i)                                                                                \
  if constexpr (i < kAChunks)                                                                     \
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint16_t *>(asrc[i]) + koff,         \
                                     sa_ + wdst + 32 * (i) * kRowBytes, 16, 0, 0);                \
  if constexpr (i < kBChunks)                                                                     \
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint16_t *>(bsrc[i]) + koff,         \
                                     sb_ + wdst + 32 * (i) * kRowBytes, 16, 0, 0);
#define GDN_ISSUE(kt, stage)                                                                      \
  do {                                                                                            \
    uint8_t *sa_ = smem + (stage) * kStage;                                                       \
    uint8_t *sb_ = sa_ + kABytes;                                                                 \
    const int koff = (kt) * kBK;                                                                  \
    GDN_REP8(GDN_DMA)                                                                             \
  } while (0)

  f32x4 acc[TM][WN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fq = lane >> 4;
  const int a_row0 = 16 * TM * wr + fr, b_row0 = 16 * WN * wc + fr;

  const int KT = K / kBK;
  if (loader) {
    // The load waves keep S - 1 k-tiles in flight: before each barrier they
    // wait for the k-tile about to be used, after it they issue the one
    // S - 1 ahead into the stage every wave has just finished with.
    for (int t = 0; t < S - 1 && t < KT; ++t) GDN_ISSUE(t, t);
    int stage = 0;
    for (int kt = 0; kt < KT; ++kt) {
      wait_vm_barrier_tiles<kLoads, S>(min(S - 2, KT - 1 - kt));
      if (kt + S - 1 < KT) GDN_ISSUE(kt + S - 1, stage == 0 ? S - 1 : stage - 1);
      stage = stage == S - 1 ? 0 : stage + 1;
    }
    return;
  }
  int stage = 0;
  for (int kt = 0; kt < KT; ++kt) {
    wait_vm_barrier<0>();                      // (a compute wave has no loads: only its LDS reads)
    const uint8_t *a = smem + stage * kStage;
    const uint8_t *b = a + kABytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 fa[TM], fb[WN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *reinterpret_cast<const bf16x8 *>(a + lds_off(a_row0 + 16 * i, 4 * ks + fq));
#pragma unroll
      for (int j = 0; j < WN; ++j)
        fb[j] = *reinterpret_cast<const bf16x8 *>(b + lds_off(b_row0 + 16 * j, 4 * ks + fq));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
    stage = stage == S - 1 ? 0 : stage + 1;
  }
#undef GDN_ISSUE
#undef GDN_DMA
#undef GDN_REP8

  gemm_epilogue<TM, WN>(g, p.M, acc, m0 + 16 * TM * wr + fr, n0 + 16 * WN * wc + 4 * fq);
}

// Tiles of 32 TM rows x 32 WN columns: tiles_m row tiles x the column tiles
// [tn0, tn0 + tiles_n), dealt to the XCDs in contiguous ranges and walked in
// groups of kGroupM row tiles. A launch whose last round of 256-row tiles
// would leave most CUs idle runs its last column tiles as a second launch of
// 128-row tiles instead (same operands, half the rows per tile).
template <int TM, int WN, int S = kStages>
__global__ __launch_bounds__(kGemmThreads) void gemm_dma_kernel(GemmParams p, int tiles_m, int tn0, int tiles_n,
                                                                int per_xcd) {
  constexpr int BM = 32 * TM, BN = 32 * WN;
  __shared__ __attribute__((aligned(16))) uint8_t smem[S * (BM + BN) * kRowBytes];
  const int logical = (blockIdx.x % kGemmXcds) * per_xcd + blockIdx.x / kGemmXcds;
  if (logical >= tiles_m * tiles_n) return;
  const int group = logical / (kGroupM * tiles_n);
  const int gm0 = group * kGroupM;
  const int gsize = min(kGroupM, tiles_m - gm0);
  const int in_group = logical - group * kGroupM * tiles_n;
  const int tm = gm0 + in_group % gsize;
  const int tn = tn0 + in_group / gsize;
  gemm_tile<TM, WN, S>(p, smem, tm * BM, tn * BN);
}

// Up to 16 rows (single-sequence decode): a block owns 16 * NF output
// columns and 16 * MF rows; its 8 waves split the contraction into
// contiguous ranges of 32-wide steps and read both operands straight into
// MFMA fragments (16 bytes per lane: the weights from HBM, the few activation
// rows from L2), U steps of loads in flight before their MFMAs; the 8 partial
// sums meet in LDS.
constexpr int kSkWaves = 8;
constexpr int kSkMaxNf = 5;
constexpr int kSkCUs = 256;

template <int MF, int NF, int U>
__global__ __launch_bounds__(kSkWaves * kWave) void gemm_skinny_kernel(GemmParams p) {
  const Segs g(p);
  const int K = p.K, M = p.M;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int fr = lane & 15, fq = lane >> 4;
  const int n0 = blockIdx.x * 16 * NF;
  const int m0 = blockIdx.y * 16 * MF;          // this block's group of rows

  // Row pointers at this lane's 8 contraction indices of a step (8 fq ..).
  u64x8 arow = {}, brow = {};
#pragma unroll
  for (int i = 0; i < MF; ++i)
    arow[i] = reinterpret_cast<uint64_t>(p.x + static_cast<int64_t>(min(m0 + 16 * i + fr, M - 1)) * K + 8 * fq);
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int n = min(n0 + 16 * j + fr, p.N - 1);
    const int s = g.seg(n);
    brow[j] = reinterpret_cast<uint64_t>(g.w(s) + static_cast<int64_t>(n - g.start(s)) * K + 8 * fq);
  }

  f32x4 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int steps = K / 32;
  const int s_lo = wave * steps / kSkWaves, s_hi = (wave + 1) * steps / kSkWaves;
  auto step = [&](int st, bf16x8 (&fa)[MF], bf16x8 (&fb)[NF]) {
#pragma unroll
    for (int i = 0; i < MF; ++i)
      fa[i] = *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const uint16_t *>(arow[i]) + 32 * st);
#pragma unroll
    for (int j = 0; j < NF; ++j)
      fb[j] = *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const uint16_t *>(brow[j]) + 32 * st);
  };
  int s0 = s_lo;
  for (; s0 + U <= s_hi; s0 += U) {
    bf16x8 fa[U][MF], fb[U][NF];
#pragma unroll
    for (int u = 0; u < U; ++u) step(s0 + u, fa[u], fb[u]);
    // Every load of the group goes out before the first MFMA waits on one.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[u][j], fa[u][i], acc[i][j], 0, 0, 0);
  }
  for (; s0 < s_hi; ++s0) {
    bf16x8 fa[MF], fb[NF];
    step(s0, fa, fb);
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int j = 0; j < NF; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  }

  // Partial sums of the waves through LDS; wave w then finishes fragments
  // f = w, w + kSkWaves, ... of the MF x NF and stores them.
  __shared__ f32x4 part[kSkWaves][MF * NF][kWave];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) part[wave][i * NF + j][lane] = acc[i][j];
  __syncthreads();
  for (int f = wave; f < MF * NF; f += kSkWaves) {
    f32x4 sum = part[0][f][lane];
#pragma unroll
    for (int w = 1; w < kSkWaves; ++w) sum += part[w][f][lane];
    const int i = f / NF, j = f % NF;
    const int m = m0 + 16 * i + fr, n = n0 + 16 * j + 4 * fq;
    const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(sum[0])) | (static_cast<uint32_t>(f32_to_bf16(sum[1])) << 16);
    const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(sum[2])) | (static_cast<uint32_t>(f32_to_bf16(sum[3])) << 16);
    if (m < M && n < g.N) {
      const int sg = g.seg(n);
      uint16_t *dst = g.out(sg) + static_cast<int64_t>(m) * g.ld(sg) + (n - g.start(sg));
      if (n + 4 <= g.end(sg) && (reinterpret_cast<uintptr_t>(dst) & 7) == 0)
        *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
      else
        store4_split(g, m, n, lo, hi);
    }
  }
}

template <int MF, int NF>
hipError_t launch_skinny(const GemmParams &p, hipStream_t s, int row_groups) {
  constexpr int U = 4;   // steps of loads in flight per wave
  const int blocks = (p.N + 16 * NF - 1) / (16 * NF);
  hipLaunchKernelGGL((gemm_skinny_kernel<MF, NF, U>), dim3(blocks, row_groups), dim3(kSkWaves * kWave), 0, s, p);
  return hipGetLastError();
}

// NF column fragments per block. A block's time is a fixed part (its walk
// of the contraction: a few round trips of loads, then the reduction through
// LDS) plus a part per fragment, fitted at about 3.7 : 1; blocks run in
// rounds of one per CU. The plan minimises rounds x (3.7 + NF).

template <int MF>
hipError_t launch_skinny_m(const GemmParams &p, hipStream_t s) {
  int best = 1;
  double best_cost = -1.0;
  for (int nf = 1; nf <= kSkMaxNf; ++nf) {
    const int64_t blocks = (p.N + 16 * nf - 1) / (16 * nf);
    const double cost = static_cast<double>((blocks + kSkCUs - 1) / kSkCUs) * (3.7 + nf);
    if (best_cost < 0 || cost < best_cost - 1e-9) {
      best_cost = cost;
      best = nf;
    }
  }
  switch (best) {
    case 1: return launch_skinny<MF, 1>(p, s, 1);
    case 2: return launch_skinny<MF, 2>(p, s, 1);
    case 3: return launch_skinny<MF, 3>(p, s, 1);
    case 4: return launch_skinny<MF, 4>(p, s, 1);
    default: return launch_skinny<MF, 5>(p, s, 1);
  }
}

struct TilePlan {
  int wn, tail_n;
};

template <int TM, int WN>
void launch_tiles(const GemmParams &p, int tiles_m, int tn0, int tiles_n, hipStream_t s) {
  const int tiles = tiles_m * tiles_n;
  if (tiles == 0) return;
  const int per_xcd = (tiles + kGemmXcds - 1) / kGemmXcds;
  hipLaunchKernelGGL((gemm_dma_kernel<TM, WN>), dim3(per_xcd * kGemmXcds), dim3(kGemmThreads), 0, s, p, tiles_m, tn0,
                     tiles_n, per_xcd);
}

template <int WN>
hipError_t launch_wn(const GemmParams &p, int tail_n, hipStream_t s) {
  constexpr int BN = 32 * WN;
  const int tiles_m = (p.M + kBM - 1) / kBM, tiles_n = (p.N + BN - 1) / BN;
  launch_tiles<kBM / 32, WN>(p, tiles_m, 0, tiles_n - tail_n, s);
  launch_tiles<kBM / 64, WN>(p, (p.M + kBM / 2 - 1) / (kBM / 2), tiles_n - tail_n, tail_n, s);
  return hipGetLastError();
}

}  // namespace

// The column-tile width, and how many of the last column tiles run as
// 128-row tiles in a second launch, are chosen per call for the least
// estimated time: rounds of 256 concurrent tiles times the tile width (plus a
// fixed cost per tile), where the round of half-height tiles costs kHalfCost
// of a full one (LDS traffic bounds these tiles, and a 128 x 160 tile moves
// 69% of a 256 x 160 tile's bytes through LDS for half its MFMA work). The
// tail is used only when the full tiles then fill whole rounds and the
// half-height ones fit in one.
constexpr int kCUs = 256;
constexpr double kHalfCost = 0.7;

static TilePlan gemm_tile_plan(int M, int N) {
  const int tiles_m = (M + kBM - 1) / kBM;
  TilePlan best{kMaxWn, 0};
  double best_cost = -1.0;
  for (int wn = kMaxWn; wn >= 4; --wn) {
    const int tiles_n = (N + 32 * wn - 1) / (32 * wn);
    const double per_round = 32.0 * wn + 16.0;
    for (int tail = 0; tail < tiles_n; ++tail) {
      const int64_t main_tiles = static_cast<int64_t>(tiles_m) * (tiles_n - tail);
      const int64_t half_tiles = 2LL * tiles_m * tail;
      if (tail > 0 && (main_tiles % kCUs != 0 || half_tiles > kCUs)) continue;
      const double cost = static_cast<double>((main_tiles + kCUs - 1) / kCUs) * per_round +
                          (tail > 0 ? kHalfCost * per_round : 0.0);
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        best = TilePlan{wn, tail};
      }
    }
  }
  return best;
}

// 17 to 64 rows (decode batches): the DMA tiles with 32 or 64 rows (TM = 1
// or 2) and 32, 64 or 96 columns (WN = 1 .. 3) and a ring of 4 k-tiles (5
// for the wider tiles: 27B out-projection 17.9 -> 16.6 us, where 32-column
// tiles lose 0.7 us with 5). The
// product is bound by the bytes each CU pulls through its vector-memory path
// (the operand rows of its tiles, once per k-tile; HBM is far from busy), so
// the shape chosen is the one with the fewest bytes on the busiest CU:
// ceil(tiles / 256) x (32 TM + 32 WN) operand rows per k-tile (ties: the
// wider tile). Measured at 64 rows against the column-split kernel below:
// 35B in-projection 19.1 -> 11.5 us, out-projection 13.0 -> 9.6 us; 27B
// 45.0 -> 30.1 and 28.8 -> 16.4 us.
template <int TM, int WN>
hipError_t launch_decode_tile(const GemmParams &p, hipStream_t s) {
  constexpr int kDecodeStages = WN == 1 ? 4 : 5;
  const int tiles_m = (p.M + 32 * TM - 1) / (32 * TM), tiles_n = (p.N + 32 * WN - 1) / (32 * WN);
  const int per_xcd = (tiles_m * tiles_n + kGemmXcds - 1) / kGemmXcds;
  hipLaunchKernelGGL((gemm_dma_kernel<TM, WN, kDecodeStages>), dim3(per_xcd * kGemmXcds), dim3(kGemmThreads), 0, s,
                     p, tiles_m, 0, tiles_n, per_xcd);
  return hipGetLastError();
}

hipError_t launch_decode(const GemmParams &p, hipStream_t s) {
  int best_tm = 1, best_wn = 1;
  int64_t best_cost = -1;
  for (int tm = 1; tm <= (p.M > 32 ? 2 : 1); ++tm)
    for (int wn = 1; wn <= 3; ++wn) {
      const int64_t tiles = static_cast<int64_t>((p.M + 32 * tm - 1) / (32 * tm)) * ((p.N + 32 * wn - 1) / (32 * wn));
      const int64_t cost = (tiles + kCUs - 1) / kCUs * (32 * tm + 32 * wn);
      if (best_cost < 0 || cost < best_cost || (cost == best_cost && wn > best_wn)) {
        best_cost = cost;
        best_tm = tm;
        best_wn = wn;
      }
    }
  if (best_tm == 2) {
    if (best_wn == 1) return launch_decode_tile<2, 1>(p, s);
    if (best_wn == 2) return launch_decode_tile<2, 2>(p, s);
    return launch_decode_tile<2, 3>(p, s);
  }
  if (best_wn == 1) return launch_decode_tile<1, 1>(p, s);
  if (best_wn == 2) return launch_decode_tile<1, 2>(p, s);
  return launch_decode_tile<1, 3>(p, s);
}

hipError_t launch_gemm(const GemmParams &p, hipStream_t s) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  if (p.M <= 16) return launch_skinny_m<1>(p, s);
  if (p.M <= 64) return launch_decode(p, s);
  const TilePlan plan = gemm_tile_plan(p.M, p.N);
  if (plan.wn == 4) return launch_wn<4>(p, plan.tail_n, s);
  return launch_wn<5>(p, plan.tail_n, s);
}

}  // namespace gdn
