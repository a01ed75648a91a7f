/*
 * gdn.h -- C ABI of the gated DeltaNet token mixer for AMD Instinct MI355X
 * (gfx950), implemented in libgdn.so.
 *
 * The mixer is the one the xwen CLAUDE.md page specifies for the Qwen 3.6
 * hybrid layers (section "Architecture cheat sheet", gated DeltaNet
 * paragraph). Its core starts from the already projected fused qkv stream and
 * ends after the gated RMSNorm; gdn_in_proj and gdn_out_proj add the bf16
 * projections before and after it (the layer input x -> qkv, z and the gate
 * logits; y -> the layer output).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers. Every buffer pointer is a DEVICE pointer (memory the caller
 * allocated on the current HIP device), except `cfg`, which is a host pointer.
 * The caller owns every buffer; the library allocates nothing and keeps no
 * state between calls. All recurrent state travels in the explicit
 * conv-state and delta-state buffers.
 *
 * Streams. `stream` is a hipStream_t passed as void* (NULL = the null
 * stream). Every call validates its arguments on the host, then enqueues its
 * kernels on `stream` and returns without synchronising. Nothing prints,
 * aborts or exits.
 *
 * Errors. A failed argument check returns GDN_E_INVALID_ARG or
 * GDN_E_UNSUPPORTED and launches nothing. A launch failure returns GDN_E_HIP.
 * Faults during kernel execution surface at the caller's next
 * synchronisation, as for any HIP kernel.
 *
 * Shapes and layouts (row-major, last index fastest). T = tokens in the call,
 * N = sequences, Hqk = K/Q heads, Hv = V heads, d = head_dim = 128,
 * C = d * (2*Hqk + Hv) = fused width.
 *   qkv            [T][C]        act dtype; q block | k block | v block, each
 *                                head-major, d contiguous channels per head
 *   beta_logit,
 *   alpha_logit    [T][Hv]       act dtype
 *   conv_w         [C][4]        fp32; conv_w[c][3] multiplies the current
 *                                token, conv_w[c][0] the token three back
 *   dt_bias, A_log [Hv]          fp32
 *   conv_state     [N][3][C]     act dtype; the 3 raw qkv rows preceding the
 *                                next token, oldest first
 *   q, k           [T][Hqk][d]   fp32; L2-normalised
 *   v              [T][Hv][d]    fp32
 *   beta, g        [T][Hv]       fp32
 *   S              [N][Hv][d][d] fp32; S[n][j][i][c], i = key index,
 *                                c = value index
 *   o              [T][Hv][d]    act dtype; delta-rule readout
 *   z, y           [T][Hv][d]    act dtype
 * V-head j uses K/Q-head j mod Hqk (tiled repeat).
 * Packed sequences: sequence n owns tokens cu_seqlens[n] .. cu_seqlens[n+1]-1;
 * cu_seqlens is a DEVICE int32 array of n_seqs+1 non-decreasing entries with
 * cu_seqlens[0] = 0 and cu_seqlens[n_seqs] = n_tokens. The library cannot
 * check its contents on the host; entries outside that contract are the
 * caller's error (kernels clamp every index they derive from it to the
 * buffers' bounds).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define GDN_API __attribute__((visibility("default")))
#else
#define GDN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_E_INVALID_ARG = 1,   /* null pointer, bad size or count, aliasing not allowed */
    GDN_E_UNSUPPORTED = 2,   /* a configuration this build does not implement */
    GDN_E_HIP = 3,           /* a HIP runtime call or kernel launch failed */
    GDN_E_WORKSPACE = 4,     /* workspace missing or smaller than required */
    GDN_E_TOO_LARGE = 5      /* more scratch needed than gdn_prefill_fused_static holds */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Form of the q/k L2 norm. GDN_L2_CLAMP is the page's canonical form
 * x / max(||x||, l2_eps); GDN_L2_RSQRT is x / sqrt(sum x^2 + l2_eps), the form
 * the page notes for the HF checkpoint (the two differ only near zero). */
typedef enum { GDN_L2_CLAMP = 0, GDN_L2_RSQRT = 1 } gdn_l2_mode;

typedef void *gdn_stream_t;  /* a hipStream_t */

typedef struct {
    int32_t n_qk_heads;      /* Hqk >= 1 */
    int32_t n_v_heads;       /* Hv >= 1, a multiple of Hqk */
    int32_t head_dim;        /* d; only 128 is implemented */
    int32_t conv_kernel;     /* only 4 is implemented */
    float l2_eps;            /* q/k L2 norm epsilon (the page: 1e-6) */
    float norm_eps;          /* gated RMSNorm epsilon (the page: 1e-6) */
    gdn_dtype act_dtype;     /* qkv, logits, conv state, o, z, y */
    gdn_l2_mode l2_mode;     /* GDN_L2_CLAMP (default) or GDN_L2_RSQRT */
} gdn_config;

/* A config with the page's values: Hqk, Hv as given, d = 128, kernel 4,
 * both epsilons 1e-6, the clamp-form L2 norm, activations of type `act`. */
GDN_API gdn_config gdn_default_config(int32_t n_qk_heads, int32_t n_v_heads, gdn_dtype act);

/*
 * gdn_conv_gate_prep -- the steps before the delta rule (the xwen CLAUDE.md
 * page, section "Architecture cheat sheet", gated DeltaNet paragraph, up to
 * the gates; the epsilon 1e-6 from the same section, the tiled V-head order
 * and ssm_a = -exp(A_log) from its section "GGUF facts that differ from the
 * HF checkpoint"):
 *   causal depthwise conv over all C fused channels, kernel 4, no bias, with
 *   the 3 rows of conv_state_in as left context of each sequence;
 *   SiLU over all C channels; split into q | k | v;
 *   q and k divided by max(||x||_2, l2_eps) per head;
 *   beta = sigmoid(beta_logit); g = -exp(A_log) * softplus(alpha_logit + dt_bias).
 * conv_state_out[n] receives the last 3 rows of [conv_state_in[n]; qkv rows
 * of sequence n] (raw inputs, copied bit for bit); a sequence with 0 tokens
 * passes its state through.
 * conv_state_out may equal conv_state_in (in-place update). No other
 * buffers may overlap. n_tokens may be 0 (only the state copy runs).
 * Decode is the case n_tokens == n_seqs with cu_seqlens = {0, 1, ..., N}.
 * Alignment: conv_w 16 bytes; qkv and both conv states two activation
 * values (4 bytes bf16, 8 bytes fp32); q, k, v 8 bytes. A misaligned
 * pointer is GDN_E_INVALID_ARG.
 */
GDN_API gdn_status gdn_conv_gate_prep(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens,
                              const int32_t *cu_seqlens,
                              const void *qkv, const void *beta_logit, const void *alpha_logit,
                              const float *conv_w, const float *dt_bias, const float *A_log,
                              const void *conv_state_in, void *conv_state_out,
                              float *q, float *k, float *v, float *beta, float *g,
                              gdn_stream_t stream);

/*
 * gdn_prefill_chunked -- the delta rule over packed sequences in its chunked
 * form (chunks of 64 tokens counted from each sequence's first token; the
 * xwen CLAUDE.md page names chunk 64 in its section "Ground truth, in order
 * of authority", and gives the recurrent step this form rewrites exactly in
 * its section "Architecture cheat sheet", gated DeltaNet paragraph).
 * Per sequence n and V-head j it produces the same result as the recurrent
 * step of gdn_decode_step applied token by token from S_in[n][j]:
 *   o[t][j] = readout after each token, S_out[n][j] = state after the last.
 * S_out may equal S_in. `workspace` is device scratch of at least
 * gdn_prefill_workspace_bytes(cfg, n_seqs, n_tokens) bytes (may be NULL
 * when that size is 0); it holds no result between calls.
 * Alignment: q, k, v 16 bytes; o four activation values (8 bytes bf16,
 * 16 bytes fp32).
 */
GDN_API gdn_status gdn_prefill_chunked(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens,
                               const int32_t *cu_seqlens,
                               const float *q, const float *k, const float *v,
                               const float *beta, const float *g,
                               const float *S_in, float *S_out, void *o,
                               void *workspace, size_t workspace_bytes, gdn_stream_t stream);

/*
 * gdn_prefill_chunked_ckpt -- gdn_prefill_chunked that also keeps the delta
 * state at block boundaries, for re-seeding later calls from a cached prefix:
 * S_ckpt [N][ckpt_cap][Hv][d][d] fp32, plane c of sequence n = S after its
 * first (c + 1) * ckpt_every tokens, written for every such boundary inside
 * the sequence (or at its end) with c < ckpt_cap; other planes are left
 * untouched. ckpt_every must be a multiple of the chunk length 64 (0, or
 * ckpt_cap = 0, writes no checkpoint). o and S_out are the same as without
 * checkpoints. S_ckpt must not overlap any other buffer. Alignment as for
 * gdn_prefill_chunked. Prefix-cache snapshots that carry the recurrent
 * state are named in the xwen CLAUDE.md page's section "serve"; the
 * serverAppConfigs commit log describes GDN states checkpointed once per
 * block of tokens and re-seeded from there, one of which went non-finite.
 */
GDN_API gdn_status gdn_prefill_chunked_ckpt(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens,
                               const int32_t *cu_seqlens, const float *q, const float *k, const float *v,
                               const float *beta, const float *g, const float *S_in, float *S_out, void *o,
                               int32_t ckpt_every, int32_t ckpt_cap, float *S_ckpt,
                               void *workspace, size_t workspace_bytes, gdn_stream_t stream);

/*
 * gdn_conv_state_ckpt -- the conv states at the same boundaries: conv_ckpt
 * [N][ckpt_cap][3][C] act dtype, plane c of sequence n = the 3 raw rows of
 * [conv_state_in[n]; its qkv rows] before token (c + 1) * ckpt_every, copied
 * bit for bit (the conv state a call resuming there needs), for every such
 * token inside the sequence or at its end, c < ckpt_cap. ckpt_every >= 1.
 * Alignment: qkv, conv_state_in and conv_ckpt two activation values.
 */
GDN_API gdn_status gdn_conv_state_ckpt(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens,
                               const int32_t *cu_seqlens, const void *qkv, const void *conv_state_in,
                               int32_t ckpt_every, int32_t ckpt_cap, void *conv_ckpt, gdn_stream_t stream);

/*
 * gdn_state_check -- a non-finite guard over n_values fp32 state values S
 * (16-byte aligned): writes stats[0] = number of NaN/Inf values and
 * stats[1] = the bit pattern of max |x| over the finite ones (a float, 0 when
 * there are none) to the device int32 array stats[2]. Nothing is returned to
 * the host: the caller reads stats after synchronising. Two kernels (one
 * clears stats), no memset, so the call can be captured in a HIP graph.
 */
GDN_API gdn_status gdn_state_check(const float *S, int64_t n_values, int32_t *stats, gdn_stream_t stream);

/*
 * gdn_prefill_fused -- the whole mixer over packed sequences (the work of
 * gdn_conv_gate_prep, gdn_prefill_chunked and gdn_gated_rmsnorm, the page's
 * gated DeltaNet paragraph in its order) without storing q, k, v, beta or g:
 * the chunked kernels compute them from the raw qkv rows and the logits as
 * they load them. Same arithmetic as the three calls; o is kept in the
 * workspace (act dtype) between the delta rule and the norm.
 *   qkv [T][C], beta_logit, alpha_logit [T][Hv], z, y [T][Hv][d]: act dtype
 *   conv_w [C][4], dt_bias, A_log [Hv], norm_w [d]: fp32
 *   conv_state_in, conv_state_out [N][3][C]: act dtype; may be the same
 *     buffer (each part of the old state is read before it is replaced)
 *   S_in, S_out [N][Hv][d][d]: fp32; may be the same buffer
 * qkv, conv_w and both conv states must be 16-byte aligned; `workspace`
 * 256-byte aligned, of gdn_prefill_fused_workspace_bytes(cfg, n_seqs,
 * n_tokens) bytes (may be NULL when that is 0). z, y and norm_w must be
 * 16-byte aligned too. Kernels on `stream`: two when the sequential pass
 * (4 blocks per sequence and V-head) leaves at least 32 of the chip's 256
 * CUs idle, whose idle CUs then form y and the new conv state as the pass
 * produces o; otherwise three, the last a norm launch that writes y and the
 * new conv state.
 */
GDN_API gdn_status gdn_prefill_fused(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens,
                             const int32_t *cu_seqlens, const void *qkv, const void *beta_logit,
                             const void *alpha_logit, const void *z, const float *conv_w, const float *dt_bias,
                             const float *A_log, const float *norm_w, const void *conv_state_in,
                             void *conv_state_out, const float *S_in, float *S_out, void *y,
                             void *workspace, size_t workspace_bytes, gdn_stream_t stream);

/*
 * gdn_prefill_fused_static -- gdn_prefill_fused without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments, arithmetic, outputs, alignment and aliasing rules as
 * gdn_prefill_fused, minus `workspace` and `workspace_bytes`.
 *
 * Its workspace is a static device array of GDN_STATIC_SCRATCH_BYTES
 * (256 MiB) in the library, one per device, which each device that loads the
 * library's code holds until the process ends. The call allocates nothing:
 * no hipMalloc, no hipFree, no allocating library routine. Its first call on
 * a device looks up that device's array (the stream, if not NULL, must belong
 * to the current device, else GDN_E_INVALID_ARG).
 *
 * Limit: gdn_prefill_fused_workspace_bytes(cfg, n_seqs, n_tokens) must not
 * exceed GDN_STATIC_SCRATCH_BYTES, else GDN_E_TOO_LARGE and nothing is
 * launched. For 16 K-heads and 48 V-heads in bf16 that admits one sequence of
 * up to 4,928 tokens (the 4,096-token prefill fits); a longer prefill
 * is split over calls, since the conv and delta states carry it across.
 *
 * Every call on a device shares that device's array and nothing in it
 * survives a call, so calls that overlap in time on one device (different
 * streams, or host threads) race and corrupt each other: serialise them.
 */
GDN_API gdn_status gdn_prefill_fused_static(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens,
                                    const int32_t *cu_seqlens, const void *qkv, const void *beta_logit,
                                    const void *alpha_logit, const void *z, const float *conv_w,
                                    const float *dt_bias, const float *A_log, const float *norm_w,
                                    const void *conv_state_in, void *conv_state_out, const float *S_in,
                                    float *S_out, void *y, gdn_stream_t stream);
#define GDN_STATIC_SCRATCH_BYTES (256u * 1024u * 1024u)

/*
 * gdn_prefill_fused_ckpt -- gdn_prefill_fused that also keeps the states at
 * block boundaries, for re-seeding later calls from a cached prefix (the same
 * planes as gdn_prefill_chunked_ckpt and gdn_conv_state_ckpt, from the fused
 * kernels):
 *   S_ckpt    [N][ckpt_cap][Hv][d][d] fp32: plane c of sequence n = S after
 *             its first (c + 1) * ckpt_every tokens
 *   conv_ckpt [N][ckpt_cap][3][C] act dtype, or NULL for none: plane c = the
 *             3 raw rows before token (c + 1) * ckpt_every (two activation
 *             values aligned)
 * for every such boundary inside the sequence or at its end with c <
 * ckpt_cap; other planes are left untouched. ckpt_every is a multiple of the
 * chunk length 64 (0, or ckpt_cap = 0, writes no checkpoint). y, S_out and the
 * new conv state are the same as without checkpoints. The planes must not
 * overlap any other buffer. Other arguments as for gdn_prefill_fused.
 */
GDN_API gdn_status gdn_prefill_fused_ckpt(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens,
                                  const int32_t *cu_seqlens, const void *qkv, const void *beta_logit,
                                  const void *alpha_logit, const void *z, const float *conv_w,
                                  const float *dt_bias, const float *A_log, const float *norm_w,
                                  const void *conv_state_in, void *conv_state_out, const float *S_in, float *S_out,
                                  void *y, int32_t ckpt_every, int32_t ckpt_cap, float *S_ckpt, void *conv_ckpt,
                                  void *workspace, size_t workspace_bytes, gdn_stream_t stream);

/* Workspace size gdn_prefill_fused needs for these sizes (0 for a bad cfg). */
GDN_API size_t gdn_prefill_fused_workspace_bytes(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens);

/* Workspace size gdn_prefill_chunked needs for these sizes (0 for a bad cfg). */
GDN_API size_t gdn_prefill_workspace_bytes(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens);

/*
 * gdn_decode_step -- one recurrent step of the delta rule for n_seqs
 * sequences of one token each (inputs laid out with T = n_seqs). Per sequence
 * n and V-head j, the recurrent step of the xwen CLAUDE.md page (section
 * "Architecture cheat sheet", gated DeltaNet paragraph), in its order:
 *   S <- exp(g) * S;  delta = beta * (v - S.k);  S <- S + k (x) delta;
 *   o = (S . q) / sqrt(head_dim)   (read from the updated state)
 * with S [128 key][128 value] fp32 per (sequence, V-head) and V-head j
 * reading q, k of K-head j mod Hqk. S_out may equal S_in (in-place update).
 * Alignment: S_in, S_out, q, k, v 16 bytes; o four activation values.
 */
GDN_API gdn_status gdn_decode_step(const gdn_config *cfg, int32_t n_seqs,
                           const float *q, const float *k, const float *v,
                           const float *beta, const float *g,
                           const float *S_in, float *S_out, void *o, gdn_stream_t stream);

/*
 * gdn_decode_fused -- one decode step of the whole mixer in a single launch,
 * for n_seqs sequences of one token each: the work of gdn_conv_gate_prep
 * (with cu_seqlens = 0, 1, .., n_seqs), gdn_decode_step and
 * gdn_gated_rmsnorm, without storing q, k, v, beta, g or o. Same arithmetic
 * as those three calls (the page's section "Architecture cheat sheet", gated
 * DeltaNet paragraph), except that the readout o reaches the norm in fp32
 * rather than rounded to the act dtype.
 *   qkv [N][C], beta_logit, alpha_logit [N][Hv], z, y [N][Hv][d]: act dtype
 *   conv_w [C][4], dt_bias [Hv], A_log [Hv], norm_w [d]: fp32
 *   conv_state_in, conv_state_out [N][3][C]: act dtype; they must NOT overlap
 *     (blocks of the step read channels of the old state that other blocks
 *     write), so a caller alternates two buffers.
 *   S_in, S_out [N][Hv][d][d]: fp32; S_out may equal S_in.
 * n_seqs may be 0. Alignment: S_in, S_out, norm_w, conv_w 16 bytes; z, y
 * four activation values; qkv and the conv states two.
 */
GDN_API gdn_status gdn_decode_fused(const gdn_config *cfg, int32_t n_seqs, const void *qkv,
                            const void *beta_logit, const void *alpha_logit, const void *z,
                            const float *conv_w, const float *dt_bias, const float *A_log,
                            const float *norm_w, const void *conv_state_in, void *conv_state_out,
                            const float *S_in, float *S_out, void *y, gdn_stream_t stream);

/*
 * gdn_decode_verify -- K = n_tokens consecutive tokens for each of n_seqs
 * sequences in one launch (a draft block under speculative decoding), with
 * the recurrent state and the conv state after EVERY token kept as snapshot
 * planes, most recent first, so that a caller that accepts only the first a
 * tokens resumes from plane K - a without recomputing (plane 0 is the state
 * after all K tokens). The arithmetic per token is that of gdn_decode_fused
 * (the page's section "Architecture cheat sheet", gated DeltaNet paragraph;
 * the page's speculative-decoding notes keep per-token state planes in this
 * most-recent-first order for the verify walk's rollback).
 *   qkv [N][K][C], beta_logit, alpha_logit [N][K][Hv], z, y [N][K][Hv][d]
 *   conv_state_in [N][3][C]           the state before the first token
 *   conv_snap [N][K][3][C]            plane p = conv state after token K-1-p
 *   S_in [N][Hv][d][d]                the state before the first token
 *   S_snap [N][K][Hv][d][d]           plane p = S after token K-1-p
 * conv_snap must not overlap conv_state_in; S_snap must not overlap S_in
 * (K = 1 may update S in place). n_seqs or n_tokens may be 0. Alignment as
 * for gdn_decode_fused (S_snap and conv_snap in place of S_out and
 * conv_state_out).
 */
GDN_API gdn_status gdn_decode_verify(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens, const void *qkv,
                             const void *beta_logit, const void *alpha_logit, const void *z,
                             const float *conv_w, const float *dt_bias, const float *A_log,
                             const float *norm_w, const void *conv_state_in, void *conv_snap,
                             const float *S_in, float *S_snap, void *y, gdn_stream_t stream);

/*
 * gdn_gated_rmsnorm -- the gated RMSNorm that ends the mixer (the xwen
 * CLAUDE.md page, section "Architecture cheat sheet", gated DeltaNet
 * paragraph: normalise, multiply by ssm_norm.weight [128], then by silu(z);
 * the epsilon 1e-6 from the same section; the weight used as stored, without
 * +1, from its section "GGUF facts that differ from the HF checkpoint"). Per
 * row of d values (n_rows = T * Hv, one row per token and V-head):
 *   y = o / sqrt(mean(o^2) + norm_eps) * norm_w * silu(z)
 * with norm_w [d] fp32 shared by all heads. y may equal o (in place); no
 * other buffers may overlap. n_rows may be 0. Alignment: o, z, y and norm_w
 * 16 bytes.
 */
GDN_API gdn_status gdn_gated_rmsnorm(const gdn_config *cfg, int64_t n_rows, const void *o, const void *z,
                             const float *norm_w, void *y, gdn_stream_t stream);

/*
 * gdn_in_proj -- the four input projections of the layer input (the page's
 * gated DeltaNet paragraph: attn_qkv, attn_gate, ssm_beta, ssm_alpha, each a
 * Linear without bias applied to x), as one bf16 product on the matrix cores:
 *   qkv = x W_qkv^T, z = x W_gate^T, beta_logit = x W_beta^T, alpha_logit = x W_alpha^T
 *   x            [T][hidden]      bf16, 16-byte aligned
 *   w_qkv        [C][hidden]      bf16, 16-byte aligned (one row per output)
 *   w_gate       [Hv*d][hidden]   bf16, 16-byte aligned
 *   w_beta,
 *   w_alpha      [Hv][hidden]     bf16, 16-byte aligned
 *   qkv [T][C], z [T][Hv][d], beta_logit, alpha_logit [T][Hv]: bf16
 * fp32 accumulation; each output rounded once to bf16 (nearest even). The
 * act dtype of cfg must be GDN_BF16 and hidden a multiple of 64 (else
 * GDN_E_UNSUPPORTED). Outputs must not overlap each other or the inputs.
 * n_tokens may be 0.
 */
GDN_API gdn_status gdn_in_proj(const gdn_config *cfg, int32_t n_tokens, int32_t hidden, const void *x,
                               const void *w_qkv, const void *w_gate, const void *w_beta, const void *w_alpha,
                               void *qkv, void *z, void *beta_logit, void *alpha_logit, gdn_stream_t stream);

/*
 * gdn_out_proj -- ssm_out, the projection after the gated RMSNorm (the page's
 * gated DeltaNet paragraph): out = y W_out^T.
 *   y      [T][Hv*d]       bf16, 16-byte aligned
 *   w_out  [hidden][Hv*d]  bf16, 16-byte aligned (one row per output)
 *   out    [T][hidden]     bf16
 * fp32 accumulation, each output rounded once to bf16. The act dtype of cfg
 * must be GDN_BF16. out must not overlap y or w_out. n_tokens may be 0.
 */
GDN_API gdn_status gdn_out_proj(const gdn_config *cfg, int32_t n_tokens, int32_t hidden, const void *y,
                                const void *w_out, void *out, gdn_stream_t stream);

/* A static, NUL-terminated description of a status code. */
GDN_API const char *gdn_status_string(gdn_status status);

/* The library's version string (static). */
GDN_API const char *gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
