// gdn_device.h -- device-side helpers shared by the gfx950 kernels of libgdn.
//
// Wave64 reductions and scans, bf16 <-> fp32 conversion, activation loads and
// stores, the scalar functions of the mixer, and the 16x16 MFMA tile step in
// the two precisions the library uses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {

// ------------------------------------------------------------ bf16 storage
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

// Activation element types: float or bf16_t.
template <typename T> struct Act;
template <> struct Act<float> {
  static __device__ __forceinline__ float load(const float *p, size_t i) { return p[i]; }
  static __device__ __forceinline__ float2 load2(const float *p, size_t i) {
    return *reinterpret_cast<const float2 *>(p + i);
  }
  static __device__ __forceinline__ void store(float *p, size_t i, float x) { p[i] = x; }
  static __device__ __forceinline__ void store2(float *p, size_t i, float2 x) {
    *reinterpret_cast<float2 *>(p + i) = x;
  }
  static __device__ __forceinline__ void store4(float *p, size_t i, float4 x) {
    *reinterpret_cast<float4 *>(p + i) = x;
  }
  static __device__ __forceinline__ float4 load4(const float *p, size_t i) {
    return *reinterpret_cast<const float4 *>(p + i);
  }
};
template <> struct Act<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t *p, size_t i) { return bf16_to_f32(p[i].bits); }
  static __device__ __forceinline__ float2 load2(const bf16_t *p, size_t i) {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(p + i);
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
  }
  static __device__ __forceinline__ void store(bf16_t *p, size_t i, float x) { p[i].bits = f32_to_bf16(x); }
  static __device__ __forceinline__ void store2(bf16_t *p, size_t i, float2 x) {
    const uint32_t w = static_cast<uint32_t>(f32_to_bf16(x.x)) | (static_cast<uint32_t>(f32_to_bf16(x.y)) << 16);
    *reinterpret_cast<uint32_t *>(p + i) = w;
  }
  static __device__ __forceinline__ void store4(bf16_t *p, size_t i, float4 x) {
    uint2 w;
    w.x = static_cast<uint32_t>(f32_to_bf16(x.x)) | (static_cast<uint32_t>(f32_to_bf16(x.y)) << 16);
    w.y = static_cast<uint32_t>(f32_to_bf16(x.z)) | (static_cast<uint32_t>(f32_to_bf16(x.w)) << 16);
    *reinterpret_cast<uint2 *>(p + i) = w;
  }
  static __device__ __forceinline__ float4 load4(const bf16_t *p, size_t i) {
    const uint2 w = *reinterpret_cast<const uint2 *>(p + i);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
  }
};

// ------------------------------------------------------ scalar functions
__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }
// log(1 + e^x) without overflow: max(x, 0) + log1p(e^-|x|).
__device__ __forceinline__ float softplusf_(float x) { return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x))); }
// SiLU x sigma(x) with the hardware reciprocal and exp: a few ulp of fp32,
// far inside what bf16 activations carry; tends to x or to -0 for large |x|.
__device__ __forceinline__ float siluf_(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// 1 / (L2 norm) of a q or k head from its sum of squares: the clamp form
// 1 / max(sqrt(ss), eps), or with rsqrt_form the form 1 / sqrt(ss + eps).
__device__ __forceinline__ float l2_inv(float ss, float eps, bool rsqrt_form) {
  return rsqrt_form ? 1.0f / sqrtf(ss + eps) : 1.0f / fmaxf(sqrtf(ss), eps);
}

// ------------------------------------------------------ wave primitives
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// x + x from another lane of the same 16-lane row, by a DPP lane pattern.
template <int kCtrl>
__device__ __forceinline__ float dpp_add(float x) {
  const int y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, true);
  return x + __builtin_bit_cast(float, y);
}

// Sum over each 16-lane row, left in every lane of the row: quad_perm
// [1,0,3,2] and [2,3,0,1] give quad sums, row_half_mirror adds the other
// quad of each 8-lane half, row_mirror adds the other half.
__device__ __forceinline__ float row16_sum(float x) {
  x = dpp_add<0xb1>(x);
  x = dpp_add<0x4e>(x);
  x = dpp_add<0x141>(x);
  x = dpp_add<0x140>(x);
  return x;
}

// Sum over the 64 lanes of the wave (every lane gets it): row sums by DPP,
// then the four rows' sums read from lanes 0, 16, 32, 48.
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (l >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ float wave_inclusive_scan_f(float x) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float y = __shfl_up(x, off, kWave);
    if (l >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ double wave_inclusive_scan_d(double x) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double y = __shfl_up(x, off, kWave);
    if (l >= off) x += y;
  }
  return x;
}

// Units (token tiles or chunks) are numbered sequence by sequence: sequence s
// owns units_of(L_s) consecutive unit ids, L_s = cu[s+1] - cu[s]. Find the
// sequence and the unit index inside it for unit id `target`, scanning
// cu_seqlens 64 sequences at a time with one wave. Returns false when the id
// is past the last unit. `min_units` is 1 when an empty sequence still owns a
// unit (the prep's conv-state copy), 0 otherwise.
__device__ __forceinline__ bool find_unit(const int *cu, int n_seqs, int target, int unit_len,
                                          int min_units, int *seq, int *unit) {
  const int l = lane_id();
  int base = 0;
  for (int s0 = 0; s0 < n_seqs; s0 += kWave) {
    const int s = s0 + l;
    int cnt = 0;
    if (s < n_seqs) {
      const int L = max(cu[s + 1] - cu[s], 0);
      cnt = max(min_units, (L + unit_len - 1) / unit_len);
    }
    const int incl = wave_inclusive_scan(cnt);
    const int excl = incl - cnt;
    const bool hit = s < n_seqs && base + excl <= target && target < base + incl;
    const unsigned long long m = __ballot(hit);
    if (m) {
      const int src = __ffsll(m) - 1;
      *seq = s0 + src;
      *unit = target - base - __shfl(excl, src, kWave);
      return true;
    }
    base += __shfl(incl, kWave - 1, kWave);
  }
  return false;
}

// Unit id of the first unit of sequence `seq` (same numbering as find_unit).
__device__ __forceinline__ int first_unit(const int *cu, int seq, int unit_len, int min_units) {
  const int l = lane_id();
  int total = 0;
  for (int s0 = 0; s0 < seq; s0 += kWave) {
    const int s = s0 + l;
    int cnt = 0;
    if (s < seq) {
      const int L = max(cu[s + 1] - cu[s], 0);
      cnt = max(min_units, (L + unit_len - 1) / unit_len);
    }
    total += wave_sum_i(cnt);
  }
  return total;
}

// ---------------------------------------------------------------- MFMA
// One 16x16 output tile, contraction depth 32 per step. Operand fragments
// follow the 16x16x32 bf16 instruction's layout for both precisions:
//   A fragment, lane l: A[row = l % 16][k = 8 * (l / 16) + e], e = 0..7
//   B fragment, lane l: B[k = 8 * (l / 16) + e][col = l % 16], e = 0..7
//   accumulator, lane l: C[row = 4 * (l / 16) + r][col = l % 16], r = 0..3
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

enum class Prec { F32, BF16X3 };

// Operands live in LDS (and in the prefill workspace) as 32-byte blocks of
// 8 consecutive contraction indices k, so that a fragment is two 16-byte
// reads with no conversion:
//   F32:    8 x fp32; the MMA issues eight 16x16x4 fp32 MFMAs, the e-th one
//           taking element e of each lane's fragment (every k once).
//   BF16X3: 8 x bf16 hi followed by 8 x bf16 lo, hi = bf16(x) and
//           lo = bf16(x - hi); the MMA sums hi*hi + hi*lo + lo*hi with three
//           16x16x32 bf16 MFMAs (the dropped lo*lo term is below 2^-16
//           relative), an fp32-grade product.
// An operand row of K contraction indices takes K/8 blocks; rows are padded
// by the caller to spread LDS banks.
constexpr int kBlk = 32;   // bytes per 8-index block

template <Prec P> struct Op;

template <> struct Op<Prec::F32> {
  struct Frag { f32x4 a, b; };
  static __device__ __forceinline__ Frag load(const uint8_t *blk) {
    Frag f;
    f.a = *reinterpret_cast<const f32x4 *>(blk);
    f.b = *reinterpret_cast<const f32x4 *>(blk + 16);
    return f;
  }
  // Four consecutive indices k .. k+3 (k % 4 == 0) of one row.
  static __device__ __forceinline__ void put4(uint8_t *row, int k, f32x4 x) {
    *reinterpret_cast<f32x4 *>(row + (k >> 3) * kBlk + (k & 7) * 4) = x;
  }
  // Element (k, idx) of a matrix stored k-major with `pitch` bytes per k row
  // and idx as the blocked index: the fragment whose tile index runs along
  // the blocked axis (a transposed read).
  static __device__ __forceinline__ Frag gather(const uint8_t *base, int pitch, int idx, int k0) {
    Frag f;
    const uint8_t *p = base + k0 * pitch + (idx >> 3) * kBlk + (idx & 7) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) f.a[e] = *reinterpret_cast<const float *>(p + e * pitch);
#pragma unroll
    for (int e = 0; e < 4; ++e) f.b[e] = *reinterpret_cast<const float *>(p + (e + 4) * pitch);
    return f;
  }
  static __device__ __forceinline__ void mma(f32x4 &c, const Frag &a, const Frag &b) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a[e], b.a[e], c, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b[e], b.b[e], c, 0, 0, 0);
  }
  static __device__ __forceinline__ void mma2(f32x4 &c0, f32x4 &c1, const Frag &a, const Frag &b0, const Frag &b1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a[e], b0.a[e], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a[e], b1.a[e], c1, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b[e], b0.b[e], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b[e], b1.b[e], c1, 0, 0, 0);
    }
  }
};

__device__ __forceinline__ void split4(f32x4 x, bf16x4 &hi, bf16x4 &lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const __bf16 h = static_cast<__bf16>(x[e]);
    hi[e] = h;
    lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(h));
  }
}

template <> struct Op<Prec::BF16X3> {
  struct Frag { bf16x8 hi, lo; };
  static __device__ __forceinline__ Frag load(const uint8_t *blk) {
    Frag f;
    f.hi = *reinterpret_cast<const bf16x8 *>(blk);
    f.lo = *reinterpret_cast<const bf16x8 *>(blk + 16);
    return f;
  }
  static __device__ __forceinline__ void put4(uint8_t *row, int k, f32x4 x) {
    bf16x4 hi, lo;
    split4(x, hi, lo);
    uint8_t *b = row + (k >> 3) * kBlk + (k & 7) * 2;
    *reinterpret_cast<bf16x4 *>(b) = hi;
    *reinterpret_cast<bf16x4 *>(b + 16) = lo;
  }
  static __device__ __forceinline__ Frag gather(const uint8_t *base, int pitch, int idx, int k0) {
    Frag f;
    const uint8_t *p = base + k0 * pitch + (idx >> 3) * kBlk + (idx & 7) * 2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f.hi[e] = *reinterpret_cast<const __bf16 *>(p + e * pitch);
      f.lo[e] = *reinterpret_cast<const __bf16 *>(p + e * pitch + 16);
    }
    return f;
  }
  static __device__ __forceinline__ void mma(f32x4 &c, const Frag &a, const Frag &b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void mma2(f32x4 &c0, f32x4 &c1, const Frag &a, const Frag &b0, const Frag &b1) {
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b0.hi, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b1.hi, c1, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b0.lo, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b1.lo, c1, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b0.hi, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b1.hi, c1, 0, 0, 0);
  }
};

// Fragment-major operand layout (global memory): the 16-row x 32-index block
// (rt, ks) of a matrix with KS contraction steps sits at byte
// (rt * KS + ks) * kFragBlk; inside it, lane l = 16 * ((k % 32) / 8) + r % 16
// owns the 8 indices k of its fragment, so that a wave loads a whole
// fragment with one coalesced 1 KB access per 16-byte plane.
//   BF16X3: hi plane at l * 16, lo plane at 1024 + l * 16
//   F32:    8 floats at l * 32
constexpr int kFragBlk = 2048;

__device__ __forceinline__ size_t frag_lane_off(int KS, int r, int k) {
  const int l = 16 * ((k & 31) >> 3) + (r & 15);
  return static_cast<size_t>((r >> 4) * KS + (k >> 5)) * kFragBlk + l * 32;   // F32 lane slot
}

template <Prec P> struct FragIO;
template <> struct FragIO<Prec::F32> {
  // The whole fragment (rt, ks) of this lane (a wave stores a block with
  // coalesced 16-byte pieces).
  static __device__ __forceinline__ void store(uint8_t *m, int KS, int rt, int ks, const Op<Prec::F32>::Frag &f) {
    uint8_t *b = m + static_cast<size_t>(rt * KS + ks) * kFragBlk + lane_id() * 32;
    *reinterpret_cast<f32x4 *>(b) = f.a;
    *reinterpret_cast<f32x4 *>(b + 16) = f.b;
  }
  // Four consecutive indices k .. k+3 (k % 4 == 0) of row r.
  static __device__ __forceinline__ void put4(uint8_t *m, int KS, int r, int k, f32x4 x) {
    *reinterpret_cast<f32x4 *>(m + frag_lane_off(KS, r, k) + (k & 7) * 4) = x;
  }
  static __device__ __forceinline__ Op<Prec::F32>::Frag load(const uint8_t *m, int KS, int rt, int ks) {
    const uint8_t *b = m + static_cast<size_t>(rt * KS + ks) * kFragBlk + lane_id() * 32;
    Op<Prec::F32>::Frag f;
    f.a = *reinterpret_cast<const f32x4 *>(b);
    f.b = *reinterpret_cast<const f32x4 *>(b + 16);
    return f;
  }
};
template <> struct FragIO<Prec::BF16X3> {
  static __device__ __forceinline__ void store(uint8_t *m, int KS, int rt, int ks, const Op<Prec::BF16X3>::Frag &f) {
    uint8_t *b = m + static_cast<size_t>(rt * KS + ks) * kFragBlk + lane_id() * 16;
    *reinterpret_cast<bf16x8 *>(b) = f.hi;
    *reinterpret_cast<bf16x8 *>(b + 1024) = f.lo;
  }
  static __device__ __forceinline__ void put4(uint8_t *m, int KS, int r, int k, f32x4 x) {
    bf16x4 hi, lo;
    split4(x, hi, lo);
    const int l = 16 * ((k & 31) >> 3) + (r & 15);
    uint8_t *b = m + static_cast<size_t>((r >> 4) * KS + (k >> 5)) * kFragBlk + l * 16 + (k & 7) * 2;
    *reinterpret_cast<bf16x4 *>(b) = hi;
    *reinterpret_cast<bf16x4 *>(b + 1024) = lo;
  }
  static __device__ __forceinline__ Op<Prec::BF16X3>::Frag load(const uint8_t *m, int KS, int rt, int ks) {
    const uint8_t *b = m + static_cast<size_t>(rt * KS + ks) * kFragBlk + lane_id() * 16;
    Op<Prec::BF16X3>::Frag f;
    f.hi = *reinterpret_cast<const bf16x8 *>(b);
    f.lo = *reinterpret_cast<const bf16x8 *>(b + 1024);
    return f;
  }
};

// Fragment of rows row0.. (lane row = row0 + l % 16), contraction step k0
// (a multiple of 32), from a blocked matrix with `pitch` bytes per row.
template <Prec P>
__device__ __forceinline__ typename Op<P>::Frag frag(const uint8_t *base, int pitch, int row0, int k0) {
  const int l = lane_id();
  return Op<P>::load(base + (row0 + (l & 15)) * pitch + ((k0 >> 3) + (l >> 4)) * kBlk);
}
// Transposed fragment: tile index idx0 + l % 16 along the blocked axis,
// contraction index along the rows.
template <Prec P>
__device__ __forceinline__ typename Op<P>::Frag frag_t(const uint8_t *base, int pitch, int idx0, int k0) {
  const int l = lane_id();
  return Op<P>::gather(base, pitch, idx0 + (l & 15), k0 + 8 * (l >> 4));
}
// Store an accumulator tile transposed: element (row0 + 4(l/16) + r, col0 + l%16)
// goes to row col0 + l%16, index row0 + 4(l/16) + r of the blocked matrix.
template <Prec P>
__device__ __forceinline__ void put_acc_t(uint8_t *base, int pitch, int row0, int col0, f32x4 acc) {
  const int l = lane_id();
  Op<P>::put4(base + (col0 + (l & 15)) * pitch, row0 + 4 * (l >> 4), acc);
}

// Accumulator element r of lane l sits at (row0 + 4*(l/16) + r, col0 + l%16).
__device__ __forceinline__ int acc_row(int r) { return 4 * (lane_id() >> 4) + r; }
__device__ __forceinline__ int acc_col() { return lane_id() & 15; }

// Workgroup barrier for LDS only: waits for this wave's LDS operations, not
// for its global loads and stores, so prefetches stay in flight across it.
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// New conv state of packed sequence n, channels c and c + 1: rows L, L+1,
// L+2 of [st_in[n]; qkv rows of the sequence] (its last 3 raw rows). The
// thread reads its 3 source rows before writing, so st_out may be st_in.
template <typename TA>
__device__ __forceinline__ void conv_state_pair(const ConvStateParams &p, int n, int c) {
  if (n >= p.n_seqs || c >= p.C) return;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  if (seq0 < 0 || L < 0 || seq0 + L > p.n_tokens) return;
  const TA *qkv = static_cast<const TA *>(p.qkv);
  const TA *st_in = static_cast<const TA *>(p.st_in);
  TA *st_out = static_cast<TA *>(p.st_out);
  const size_t st_base = static_cast<size_t>(n) * (kConvK - 1) * p.C;
  float2 v[kConvK - 1];
#pragma unroll
  for (int r = 0; r < kConvK - 1; ++r) {
    const int src = L + r;   // row of [state; x]
    v[r] = src < kConvK - 1 ? Act<TA>::load2(st_in, st_base + static_cast<size_t>(src) * p.C + c)
                            : Act<TA>::load2(qkv, static_cast<size_t>(seq0 + src - (kConvK - 1)) * p.C + c);
  }
#pragma unroll
  for (int r = 0; r < kConvK - 1; ++r) Act<TA>::store2(st_out, st_base + static_cast<size_t>(r) * p.C + c, v[r]);
}

// Legacy fp32 fragments from row-major fp32 LDS (used by the small fp32 MFMA
// steps of the triangular solve).
}  // namespace gdn
