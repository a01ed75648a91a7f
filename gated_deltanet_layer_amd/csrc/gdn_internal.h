// gdn_internal.h -- host-side launch interface between the C ABI (api.hip)
// and the kernel files. Every launcher enqueues on `stream` and returns the
// launch status; argument checking has already been done by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

constexpr int kWave = 64;      // wavefront width on CDNA
constexpr int kHeadDim = 128;  // the only head dim the page's models use
constexpr int kConvK = 4;      // conv kernel size

// Token tile of the prep kernel: 32 tokens when sequences average at least
// that many (the 3-row halo is re-read once per tile), else 8 (decode-like
// calls, where a longer tile would load rows it never uses).
inline int prep_tile(int n_seqs, int n_tokens) {
  return static_cast<int64_t>(n_tokens) >= 32 * static_cast<int64_t>(n_seqs) ? 32 : 8;
}
// Chunk length of the chunked delta rule.
constexpr int kChunk = 64;

struct PrepParams {
  const int32_t *cu;
  int n_seqs, n_tokens, n_qk, n_v;
  const void *qkv, *b, *a;
  const float *conv_w, *dt_bias, *A_log;
  const void *st_in;
  void *st_out;
  float *q, *k, *v, *beta, *g;
  float l2_eps;
  int l2_mode;   // gdn_l2_mode
};
hipError_t launch_prep(const PrepParams &p, gdn_dtype act, hipStream_t s);

struct DecodeParams {
  int n_seqs, n_qk, n_v;
  const float *q, *k, *v, *beta, *g;
  const float *S_in;
  float *S_out;
  void *o;
};
hipError_t launch_decode(const DecodeParams &p, gdn_dtype act, hipStream_t s);

// n_tok tokens per sequence ([N][n_tok] rows of qkv, z, y, logits); the
// state and conv state after token t go to plane n_tok - 1 - t of S_out and
// st_out (most recent first; n_tok = 1 is a plain decode step).
struct FusedDecodeParams {
  int n_seqs, n_tok, n_qk, n_v;
  const void *qkv, *b, *a, *z;
  const float *conv_w, *dt_bias, *A_log, *norm_w;
  const void *st_in;
  void *st_out;
  const float *S_in;
  float *S_out;
  void *y;
  float l2_eps, norm_eps;
  int l2_mode;   // gdn_l2_mode
};
hipError_t launch_decode_fused(const FusedDecodeParams &p, gdn_dtype act, hipStream_t s);

struct NormParams {
  int64_t n_rows;
  const void *o, *z;
  const float *w;
  void *y;
  float eps;
};
hipError_t launch_norm(const NormParams &p, gdn_dtype act, hipStream_t s);

// Conv-state checkpoints: conv_ckpt[n][c] = the 3 raw rows before token
// (c + 1) * every of sequence n (rows of [conv_state_in; qkv]), c < cap,
// for every such token inside the sequence or at its end.
struct ConvCkptParams {
  const int32_t *cu;
  int n_seqs, n_tokens, n_qk, n_v, every, cap;
  const void *qkv, *st_in;
  void *ckpt;
};
hipError_t launch_conv_ckpt(const ConvCkptParams &p, gdn_dtype act, hipStream_t s);

// New conv states after packed sequences: conv_out[n] = the last 3 rows of
// [st_in[n]; qkv rows of sequence n] (one thread owns a channel's 3 rows, so
// st_out may equal st_in).
struct ConvStateParams {
  const int32_t *cu;
  int n_seqs, n_tokens, C;
  const void *qkv, *st_in;
  void *st_out;
};
// The gated RMSNorm and the new conv states in one launch (the states after
// the norm's blocks).
hipError_t launch_norm_conv_state(const NormParams &p, const ConvStateParams &cp, gdn_dtype act, hipStream_t s);

// Non-finite guard over n_values fp32 state values: stats[0] = number of
// non-finite values, stats[1] = bit pattern of max |x| over the finite ones.
hipError_t launch_state_check(const float *S, int64_t n_values, int32_t *stats, hipStream_t s);

// bf16 product out[m][n] = sum_k x[m][k] w[n][k] (fp32 accumulation, bf16
// out). Columns [start[s], start[s+1]) (start[n_seg] = N) form segment s: its
// weight rows come from w[s] (row n - start[s], K values each) and its outputs
// go to out[s][m * ld[s] + n - start[s]]. K is a multiple of 64; x and every
// w[s] are 16-byte aligned.
constexpr int kMaxSeg = 4;
struct GemmParams {
  int M, N, K;
  const uint16_t *x;
  int n_seg;
  int start[kMaxSeg];
  const uint16_t *w[kMaxSeg];
  uint16_t *out[kMaxSeg];
  int64_t ld[kMaxSeg];
};
hipError_t launch_gemm(const GemmParams &p, hipStream_t s);

struct PrefillParams {
  const int32_t *cu;
  int n_seqs, n_tokens, n_qk, n_v;
  const float *q, *k, *v, *beta, *g;
  const float *S_in;
  float *S_out;
  void *o;
  void *ws;
  size_t ws_bytes;
  // State checkpoints: plane c of sequence n (S_ckpt[n][c], c < ckpt_cap)
  // holds S after token (c + 1) * 64 * ckpt_chunks of the sequence, for
  // every such token inside it; ckpt_chunks = 0 writes none.
  float *S_ckpt;
  int ckpt_chunks, ckpt_cap;
  // Fused form (gdn_prefill_fused), when qkv is not null: the chunk kernels
  // compute q, k (conv, SiLU, L2 norm), v (conv, SiLU), beta and g themselves
  // from the raw qkv rows (left context: st_in) and the logits, instead of
  // reading q, k, v, beta, g.
  const void *qkv, *bl, *al, *st_in;
  const float *conv_w, *dt_bias, *A_log;
  float l2_eps;
  int l2_mode;
  // Fused form with the gated RMSNorm folded into chunk_state (fold_blocks >
  // 0): fold_blocks extra blocks of that launch form y from o, z and norm_w
  // as the slab blocks finish each (chunk, V-head); ready holds one counter
  // per (chunk, V-head), zeroed by chunk_local.
  const void *z;
  const float *norm_w;
  void *y;
  float norm_eps;
  uint32_t *ready;
  int fold_blocks;
  void *st_out;        // the new conv states (may be st_in)
};
// Upper bound on the number of chunks over all sequences.
inline int64_t max_chunks(int n_seqs, int n_tokens) {
  return (static_cast<int64_t>(n_tokens) + kChunk - 1) / kChunk + n_seqs;
}
size_t prefill_workspace_bytes(int n_seqs, int n_tokens, int n_qk, int n_v);
// uint32 words per ready counter of the folded norm (one 128-byte line each).
constexpr int kReadyStride = 32;
// Blocks of the folded norm for a fused prefill over n_seqs sequences and
// n_v V-heads: the CUs the sequential kernel leaves idle, or 0 (the norm then
// runs as a launch of its own).
int prefill_fold_blocks(int n_seqs, int n_v);
hipError_t launch_prefill(const PrefillParams &p, gdn_dtype act, hipStream_t s);

}  // namespace gdn
