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
};

// ------------------------------------------------------ scalar functions
__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }
// log(1 + e^x) without overflow: max(x, 0) + log1p(e^-|x|).
__device__ __forceinline__ float softplusf_(float x) { return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x))); }
__device__ __forceinline__ float siluf_(float x) { return x / (1.0f + expf(-x)); }

// ------------------------------------------------------ wave primitives
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
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
// F32 precision issues eight 16x16x4 fp32 MFMAs, the e-th taking element e
// of each lane's fragment (so every k of the step is covered once).
// BF16X3 splits each fp32 operand into hi = bf16(x) and lo = bf16(x - hi)
// and sums hi*hi + hi*lo + lo*hi with three 16x16x32 bf16 MFMAs; the
// dropped lo*lo term is below 2^-16 relative.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum class Prec { F32, BF16X3 };

struct Frag { float e[8]; };

template <Prec P> struct Mma;

template <> struct Mma<Prec::F32> {
  static __device__ __forceinline__ void run(f32x4 &acc, const Frag &a, const Frag &b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.e[e], b.e[e], acc, 0, 0, 0);
  }
};

__device__ __forceinline__ void split_bf16(const Frag &x, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = static_cast<__bf16>(x.e[e]);
    hi[e] = h;
    lo[e] = static_cast<__bf16>(x.e[e] - static_cast<float>(h));
  }
}

template <> struct Mma<Prec::BF16X3> {
  static __device__ __forceinline__ void run(f32x4 &acc, const Frag &a, const Frag &b) {
    bf16x8 ah, al, bh, bl;
    split_bf16(a, ah, al);
    split_bf16(b, bh, bl);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
  }
};

// Fragment loads from LDS (fp32).
// Row-major source with k contiguous: A[row][k] at base[row * ld + k].
__device__ __forceinline__ Frag frag_rows(const float *base, int ld, int row0, int k0) {
  const int l = lane_id();
  const float *p = base + (row0 + (l & 15)) * ld + k0 + 8 * (l >> 4);
  const float4 x = *reinterpret_cast<const float4 *>(p);
  const float4 y = *reinterpret_cast<const float4 *>(p + 4);
  Frag f;
  f.e[0] = x.x; f.e[1] = x.y; f.e[2] = x.z; f.e[3] = x.w;
  f.e[4] = y.x; f.e[5] = y.y; f.e[6] = y.z; f.e[7] = y.w;
  return f;
}
// Source with the tile's index (row of A, or column of B) contiguous and k
// strided: X[k][idx] at base[k * ld + idx]. Optional per-k scale.
__device__ __forceinline__ Frag frag_cols(const float *base, int ld, int idx0, int k0) {
  const int l = lane_id();
  const float *p = base + (k0 + 8 * (l >> 4)) * ld + idx0 + (l & 15);
  Frag f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.e[e] = p[e * ld];
  return f;
}
__device__ __forceinline__ Frag frag_cols_scaled(const float *base, int ld, int idx0, int k0,
                                                 const float *kscale) {
  const int l = lane_id();
  const int kb = k0 + 8 * (l >> 4);
  const float *p = base + kb * ld + idx0 + (l & 15);
  Frag f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.e[e] = p[e * ld] * kscale[kb + e];
  return f;
}

// Accumulator element r of lane l sits at (row0 + 4*(l/16) + r, col0 + l%16).
__device__ __forceinline__ int acc_row(int r) { return 4 * (lane_id() >> 4) + r; }
__device__ __forceinline__ int acc_col() { return lane_id() & 15; }

}  // namespace gdn
