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
// Tiling for gfx950. A block of 4 waves owns a kBM x BN tile (BN = 32 * WN);
// wave (wr, wc) owns rows 128 wr .. +127 and columns 16 WN wc .. +16 WN - 1,
// i.e. 8 x WN accumulator tiles of 16 x 16 (v_mfma_f32_16x16x32_bf16). The
// contraction runs in k-tiles of 64: both operand tiles are staged in LDS,
// double-buffered, one barrier per k-tile, with the next k-tile's global loads
// in flight during the current one's MFMAs. An LDS row is the 128 bytes of one
// operand row in a k-tile, as 8 chunks of 16 bytes (8 k values); chunk c of
// row r is stored at slot c ^ (r & 7), which makes both the 16-byte stores
// and the 16-byte fragment reads free of bank conflicts.
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
constexpr int kGemmThreads = 256;
constexpr int kGroupM = 4;        // row tiles per group in the tile walk
constexpr int kGemmXcds = 8;

__device__ __forceinline__ int seg_of(const GemmParams &p, int n) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < kMaxSeg; ++i)
    if (i < p.n_seg && n >= p.start[i]) s = i;
  return s;
}

// Element s of a kernel-argument array, selected with constant indices (a
// dynamic index would copy the array to private memory).
template <typename T>
__device__ __forceinline__ T pick(const T (&a)[kMaxSeg], int s) {
  T r = a[0];
#pragma unroll
  for (int i = 1; i < kMaxSeg; ++i)
    if (s == i) r = a[i];
  return r;
}

// Byte offset of chunk c of LDS row r.
__device__ __forceinline__ int lds_off(int r, int c) { return r * kRowBytes + ((c ^ (r & 7)) << 4); }

template <int WN>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmParams p, int tiles_m, int tiles_n, int per_xcd) {
  constexpr int BN = 32 * WN;
  constexpr int kAChunks = kBM * 8 / kGemmThreads;    // 16-byte chunks per thread and k-tile
  constexpr int kBChunks = BN * 8 / kGemmThreads;
  constexpr int kABytes = kBM * kRowBytes, kBBytes = BN * kRowBytes;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (kABytes + kBBytes)];

  // Tile of this block.
  const int logical = (blockIdx.x % kGemmXcds) * per_xcd + blockIdx.x / kGemmXcds;
  if (logical >= tiles_m * tiles_n) return;
  const int group = logical / (kGroupM * tiles_n);
  const int gm0 = group * kGroupM;
  const int gsize = min(kGroupM, tiles_m - gm0);
  const int in_group = logical - group * kGroupM * tiles_n;
  const int tm = gm0 + in_group % gsize;
  const int tn = in_group / gsize;
  const int m0 = tm * kBM, n0 = tn * BN;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int wr = wave >> 1, wc = wave & 1;
  const int K = p.K;

  // Global sources of this thread's chunks: row (tid >> 3) + 32 i, chunk tid & 7.
  const int lrow = tid >> 3, lchunk = tid & 7;
  const uint16_t *asrc[kAChunks];
  const uint16_t *bsrc[kBChunks];
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    const int m = min(m0 + lrow + 32 * i, p.M - 1);
    asrc[i] = p.x + static_cast<int64_t>(m) * K + 8 * lchunk;
  }
#pragma unroll
  for (int i = 0; i < kBChunks; ++i) {
    const int n = min(n0 + lrow + 32 * i, p.N - 1);
    const int s = seg_of(p, n);
    bsrc[i] = pick(p.w, s) + static_cast<int64_t>(n - pick(p.start, s)) * K + 8 * lchunk;
  }
  const int st_off = lds_off(lrow, lchunk);   // + 32 i rows (same slot: 32 i is a multiple of 8)

  uint4 ra[kAChunks], rb[kBChunks];
  auto load = [&](int kt) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) ra[i] = *reinterpret_cast<const uint4 *>(asrc[i] + kt * kBK);
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) rb[i] = *reinterpret_cast<const uint4 *>(bsrc[i] + kt * kBK);
  };
  auto store = [&](int buf) {
    uint8_t *a = smem + buf * (kABytes + kBBytes);
    uint8_t *b = a + kABytes;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) *reinterpret_cast<uint4 *>(a + st_off + 32 * i * kRowBytes) = ra[i];
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) *reinterpret_cast<uint4 *>(b + st_off + 32 * i * kRowBytes) = rb[i];
  };

  f32x4 acc[8][WN];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fragment reads: row 16 f + (lane & 15) of the wave's rows, chunk 4 ks + (lane >> 4).
  const int fr = lane & 15, fq = lane >> 4;
  const int a_row0 = 128 * wr + fr, b_row0 = 16 * WN * wc + fr;

  const int KT = K / kBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load(kt + 1);
    const uint8_t *a = smem + cur * (kABytes + kBBytes);
    const uint8_t *b = a + kABytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 fa[8], fb[WN];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        fa[i] = *reinterpret_cast<const bf16x8 *>(a + lds_off(a_row0 + 16 * i, 4 * ks + fq));
#pragma unroll
      for (int j = 0; j < WN; ++j)
        fb[j] = *reinterpret_cast<const bf16x8 *>(b + lds_off(b_row0 + 16 * j, 4 * ks + fq));
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds out[m][n .. n+3], m = row 16 i + (lane & 15), n = col 16 j + 4 (lane >> 4).
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = m0 + 128 * wr + 16 * i + fr;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int n = n0 + 16 * WN * wc + 16 * j + 4 * fq;
      if (n >= p.N) continue;
      const int s = seg_of(p, n);
      const int e0 = n - pick(p.start, s);
      const int end = s + 1 < p.n_seg ? pick(p.start, s + 1) : p.N;
      uint16_t *dst = pick(p.out, s) + static_cast<int64_t>(m) * pick(p.ld, s) + e0;
      const uint16_t h0 = f32_to_bf16(acc[i][j][0]), h1 = f32_to_bf16(acc[i][j][1]);
      const uint16_t h2 = f32_to_bf16(acc[i][j][2]), h3 = f32_to_bf16(acc[i][j][3]);
      if (n + 4 <= end && (reinterpret_cast<uintptr_t>(dst) & 7) == 0) {
        uint2 v;
        v.x = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
        v.y = static_cast<uint32_t>(h2) | (static_cast<uint32_t>(h3) << 16);
        *reinterpret_cast<uint2 *>(dst) = v;
      } else {
        const uint16_t h[4] = {h0, h1, h2, h3};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ne = n + e;
          if (ne < p.N) {
            const int se = seg_of(p, ne);
            pick(p.out, se)[static_cast<int64_t>(m) * pick(p.ld, se) + (ne - pick(p.start, se))] = h[e];
          }
        }
      }
    }
  }
}

template <int WN>
hipError_t launch_wn(const GemmParams &p, hipStream_t s) {
  constexpr int BN = 32 * WN;
  const int tiles_m = (p.M + kBM - 1) / kBM, tiles_n = (p.N + BN - 1) / BN;
  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + kGemmXcds - 1) / kGemmXcds;
  hipLaunchKernelGGL(gemm_kernel<WN>, dim3(per_xcd * kGemmXcds), dim3(kGemmThreads), 0, s, p, tiles_m, tiles_n,
                     per_xcd);
  return hipGetLastError();
}

}  // namespace

// The column-tile width is chosen per call so that the number of rounds of
// 256 concurrent tiles, times the tile width, is smallest (the last round of
// a launch is often partly idle). Wider tiles than 5 fragments per wave do
// not fit the registers next to the staging of the next k-tile.
static int gemm_tile_wn(int M, int N) {
  const int tiles_m = (M + kBM - 1) / kBM;
  int best = 5;
  int64_t best_cost = -1;
  for (int wn = 5; wn >= 4; --wn) {
    const int64_t tiles = static_cast<int64_t>(tiles_m) * ((N + 32 * wn - 1) / (32 * wn));
    const int64_t rounds = (tiles + 255) / 256;
    const int64_t cost = rounds * (32 * wn + 16);   // + a fixed per-tile cost
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = wn; }
  }
  return best;
}

hipError_t launch_gemm(const GemmParams &p, hipStream_t s) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  if (gemm_tile_wn(p.M, p.N) == 4) return launch_wn<4>(p, s);
  return launch_wn<5>(p, s);
}

}  // namespace gdn
