// api.hip -- the C ABI declared in include/gdn.h: host-side argument checks,
// then asynchronous launches on the caller's stream. Nothing here allocates,
// synchronises, prints or aborts.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

using gdn::kHeadDim;

constexpr int64_t kMaxGrid = 0x7fffffff;

bool finite_nonneg(float x) { return isfinite(x) && x >= 0.0f; }

gdn_status check_config(const gdn_config *cfg) {
  if (!cfg) return GDN_E_INVALID_ARG;
  if (cfg->n_qk_heads < 1 || cfg->n_v_heads < 1) return GDN_E_INVALID_ARG;
  if (cfg->n_v_heads % cfg->n_qk_heads != 0) return GDN_E_INVALID_ARG;
  if (cfg->act_dtype != GDN_F32 && cfg->act_dtype != GDN_BF16) return GDN_E_INVALID_ARG;
  if (cfg->l2_mode != GDN_L2_CLAMP && cfg->l2_mode != GDN_L2_RSQRT) return GDN_E_INVALID_ARG;
  if (!finite_nonneg(cfg->l2_eps) || !finite_nonneg(cfg->norm_eps)) return GDN_E_INVALID_ARG;
  if (cfg->head_dim != kHeadDim) return GDN_E_UNSUPPORTED;
  if (cfg->conv_kernel != gdn::kConvK) return GDN_E_UNSUPPORTED;
  // Grid y of the prep kernel is the number of 128-channel head blocks.
  if (2LL * cfg->n_qk_heads + cfg->n_v_heads > 65535) return GDN_E_UNSUPPORTED;
  return GDN_OK;
}

size_t act_size(const gdn_config *cfg) { return cfg->act_dtype == GDN_BF16 ? 2 : 4; }

// [a, a + na) and [b, b + nb) overlap (byte ranges; null or empty never does).
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

struct Range {
  const void *p;
  size_t n;
};

// Any overlap among the outputs, or between an output and an input.
template <size_t NO, size_t NI>
bool any_overlap(const Range (&outs)[NO], const Range (&ins)[NI]) {
  for (size_t i = 0; i < NO; ++i) {
    for (size_t j = i + 1; j < NO; ++j)
      if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return true;
    for (size_t j = 0; j < NI; ++j)
      if (overlap(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return true;
  }
  return false;
}

gdn_status launched(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_E_HIP; }

bool aligned(const void *p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// Alignment a pointer needs for the widest vector access a kernel makes
// through it (null pointers are checked elsewhere and pass here).
struct Align {
  const void *p;
  size_t a;
};
template <size_t N>
bool all_aligned(const Align (&v)[N]) {
  for (size_t i = 0; i < N; ++i)
    if (!aligned(v[i].p, v[i].a)) return false;
  return true;
}

}  // namespace

extern "C" {

gdn_config gdn_default_config(int32_t n_qk_heads, int32_t n_v_heads, gdn_dtype act) {
  gdn_config c;
  c.n_qk_heads = n_qk_heads;
  c.n_v_heads = n_v_heads;
  c.head_dim = kHeadDim;
  c.conv_kernel = gdn::kConvK;
  c.l2_eps = 1e-6f;
  c.norm_eps = 1e-6f;
  c.act_dtype = act;
  c.l2_mode = GDN_L2_CLAMP;
  return c;
}

const char *gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_E_INVALID_ARG: return "invalid argument";
    case GDN_E_UNSUPPORTED: return "unsupported configuration";
    case GDN_E_HIP: return "HIP launch or runtime error";
    case GDN_E_WORKSPACE: return "workspace missing or too small";
    case GDN_E_TOO_LARGE: return "the call needs more scratch than the static scratch holds (split the tokens over calls)";
  }
  return "unknown status";
}

const char *gdn_version(void) { return "gdn-mi355x 0.1 (gfx950)"; }

gdn_status gdn_conv_gate_prep(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens,
                              const int32_t *cu_seqlens, const void *qkv, const void *beta_logit,
                              const void *alpha_logit, const float *conv_w, const float *dt_bias,
                              const float *A_log, const void *conv_state_in, void *conv_state_out,
                              float *q, float *k, float *v, float *beta, float *g,
                              gdn_stream_t stream) {
  const gdn_status cs = check_config(cfg);
  if (cs != GDN_OK) return cs;
  if (n_seqs < 0 || n_tokens < 0) return GDN_E_INVALID_ARG;
  if (n_seqs == 0) return n_tokens == 0 ? GDN_OK : GDN_E_INVALID_ARG;
  if (!cu_seqlens || !conv_w || !dt_bias || !A_log || !conv_state_in || !conv_state_out)
    return GDN_E_INVALID_ARG;
  if (n_tokens > 0 && (!qkv || !beta_logit || !alpha_logit || !q || !k || !v || !beta || !g))
    return GDN_E_INVALID_ARG;
  const int Hqk = cfg->n_qk_heads, Hv = cfg->n_v_heads;
  const size_t C = static_cast<size_t>(kHeadDim) * (2 * Hqk + Hv);
  const size_t T = static_cast<size_t>(n_tokens), as = act_size(cfg);
  // Pairs of channels per access (qkv, conv states, q, k, v), four taps per
  // channel (conv_w).
  const Align al[] = {{qkv, 2 * as}, {conv_state_in, 2 * as}, {conv_state_out, 2 * as}, {conv_w, 16},
                      {q, 8}, {k, 8}, {v, 8}};
  if (!all_aligned(al)) return GDN_E_INVALID_ARG;
  const int tile = gdn::prep_tile(n_seqs, n_tokens);
  const int64_t tiles = (static_cast<int64_t>(n_tokens) + tile - 1) / tile + n_seqs;
  if (tiles > kMaxGrid) return GDN_E_UNSUPPORTED;
  const size_t st = static_cast<size_t>(n_seqs) * (gdn::kConvK - 1) * C * as;
  const Range outs[] = {{q, T * Hqk * kHeadDim * 4}, {k, T * Hqk * kHeadDim * 4}, {v, T * Hv * kHeadDim * 4},
                        {beta, T * Hv * 4}, {g, T * Hv * 4}};
  const Range ins[] = {{qkv, T * C * as}, {beta_logit, T * Hv * as}, {alpha_logit, T * Hv * as},
                       {conv_w, C * 4 * 4}, {dt_bias, Hv * 4u}, {A_log, Hv * 4u},
                       {cu_seqlens, (n_seqs + 1u) * 4u}, {conv_state_in, st}, {conv_state_out, st}};
  if (any_overlap(outs, ins)) return GDN_E_INVALID_ARG;
  // The conv state may be updated in place, but must not partly overlap.
  if (conv_state_in != conv_state_out && overlap(conv_state_in, st, conv_state_out, st)) return GDN_E_INVALID_ARG;
  for (const Range &r : ins)
    if (r.p != conv_state_out && r.p != conv_state_in && overlap(r.p, r.n, conv_state_out, st)) return GDN_E_INVALID_ARG;

  gdn::PrepParams p;
  p.cu = cu_seqlens;
  p.n_seqs = n_seqs;
  p.n_tokens = n_tokens;
  p.n_qk = Hqk;
  p.n_v = Hv;
  p.qkv = qkv;
  p.b = beta_logit;
  p.a = alpha_logit;
  p.conv_w = conv_w;
  p.dt_bias = dt_bias;
  p.A_log = A_log;
  p.st_in = conv_state_in;
  p.st_out = conv_state_out;
  p.q = q;
  p.k = k;
  p.v = v;
  p.beta = beta;
  p.g = g;
  p.l2_eps = cfg->l2_eps;
  p.l2_mode = cfg->l2_mode;
  return launched(gdn::launch_prep(p, cfg->act_dtype, static_cast<hipStream_t>(stream)));
}

size_t gdn_prefill_workspace_bytes(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens) {
  if (check_config(cfg) != GDN_OK || n_seqs < 0 || n_tokens < 0) return 0;
  if (n_tokens == 0) return 0;
  return gdn::prefill_workspace_bytes(n_seqs, n_tokens, cfg->n_qk_heads, cfg->n_v_heads);
}

gdn_status gdn_prefill_chunked_ckpt(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens,
                                    const int32_t *cu_seqlens, const float *q, const float *k, const float *v,
                                    const float *beta, const float *g, const float *S_in, float *S_out, void *o,
                                    int32_t ckpt_every, int32_t ckpt_cap, float *S_ckpt,
                                    void *workspace, size_t workspace_bytes, gdn_stream_t stream) {
  const gdn_status cs = check_config(cfg);
  if (cs != GDN_OK) return cs;
  if (n_seqs < 0 || n_tokens < 0) return GDN_E_INVALID_ARG;
  if (n_seqs == 0) return n_tokens == 0 ? GDN_OK : GDN_E_INVALID_ARG;
  if (!cu_seqlens || !S_in || !S_out) return GDN_E_INVALID_ARG;
  if (n_tokens > 0 && (!q || !k || !v || !beta || !g || !o)) return GDN_E_INVALID_ARG;
  if (ckpt_every < 0 || ckpt_cap < 0 || ckpt_every % gdn::kChunk != 0) return GDN_E_INVALID_ARG;
  const bool ckpt = ckpt_every > 0 && ckpt_cap > 0;
  if (ckpt && !S_ckpt) return GDN_E_INVALID_ARG;
  const int Hqk = cfg->n_qk_heads, Hv = cfg->n_v_heads;
  // q, k, v rows are read 4 floats at a time; o is written 4 values at a time.
  const Align al[] = {{q, 16}, {k, 16}, {v, 16}, {o, 4 * act_size(cfg)}};
  if (!all_aligned(al)) return GDN_E_INVALID_ARG;
  const size_t need = gdn_prefill_workspace_bytes(cfg, n_seqs, n_tokens);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_E_WORKSPACE;
  const int64_t chunks = gdn::max_chunks(n_seqs, n_tokens);
  if (chunks > kMaxGrid || Hqk > 65535 ||
      static_cast<int64_t>(n_seqs) * Hv * (kHeadDim / 32) > kMaxGrid)
    return GDN_E_UNSUPPORTED;
  const size_t T = static_cast<size_t>(n_tokens);
  const size_t sb = static_cast<size_t>(n_seqs) * Hv * kHeadDim * kHeadDim * 4;
  const Range outs[] = {{o, T * Hv * kHeadDim * act_size(cfg)}, {workspace, need}};
  const Range ins[] = {{q, T * Hqk * kHeadDim * 4}, {k, T * Hqk * kHeadDim * 4}, {v, T * Hv * kHeadDim * 4},
                       {beta, T * Hv * 4}, {g, T * Hv * 4}, {cu_seqlens, (n_seqs + 1u) * 4u},
                       {S_in, sb}, {S_out, sb}};
  if (any_overlap(outs, ins)) return GDN_E_INVALID_ARG;
  if (S_in != S_out && overlap(S_in, sb, S_out, sb)) return GDN_E_INVALID_ARG;
  for (size_t i = 0; i < 6; ++i)
    if (overlap(ins[i].p, ins[i].n, S_out, sb)) return GDN_E_INVALID_ARG;
  if (ckpt) {
    const size_t cb = static_cast<size_t>(n_seqs) * ckpt_cap * Hv * kHeadDim * kHeadDim * 4;
    for (const Range &r : ins)
      if (overlap(r.p, r.n, S_ckpt, cb)) return GDN_E_INVALID_ARG;
    if (overlap(o, T * Hv * kHeadDim * act_size(cfg), S_ckpt, cb) || overlap(workspace, need, S_ckpt, cb))
      return GDN_E_INVALID_ARG;
  }

  gdn::PrefillParams p = {};
  p.cu = cu_seqlens;
  p.n_seqs = n_seqs;
  p.n_tokens = n_tokens;
  p.n_qk = Hqk;
  p.n_v = Hv;
  p.q = q;
  p.k = k;
  p.v = v;
  p.beta = beta;
  p.g = g;
  p.S_in = S_in;
  p.S_out = S_out;
  p.o = o;
  p.ws = workspace;
  p.ws_bytes = workspace_bytes;
  p.S_ckpt = ckpt ? S_ckpt : nullptr;
  p.ckpt_chunks = ckpt ? ckpt_every / gdn::kChunk : 0;
  p.ckpt_cap = ckpt ? ckpt_cap : 0;
  return launched(gdn::launch_prefill(p, cfg->act_dtype, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_prefill_chunked(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens,
                               const int32_t *cu_seqlens, const float *q, const float *k, const float *v,
                               const float *beta, const float *g, const float *S_in, float *S_out, void *o,
                               void *workspace, size_t workspace_bytes, gdn_stream_t stream) {
  return gdn_prefill_chunked_ckpt(cfg, n_seqs, n_tokens, cu_seqlens, q, k, v, beta, g, S_in, S_out, o, 0, 0,
                                  nullptr, workspace, workspace_bytes, stream);
}

// Workspace of the fused prefill: the chunked form's, then o (act dtype),
// 256-byte aligned.
static size_t fused_o_offset(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens) {
  const size_t base = gdn::prefill_workspace_bytes(n_seqs, n_tokens, cfg->n_qk_heads, cfg->n_v_heads);
  return (base + 255) / 256 * 256;
}

// Then the folded norm's counters, one uint32 per (chunk, V-head), 256-byte
// aligned.
static size_t fused_ready_offset(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens) {
  const size_t end = fused_o_offset(cfg, n_seqs, n_tokens) +
                     static_cast<size_t>(n_tokens) * cfg->n_v_heads * kHeadDim * act_size(cfg);
  return (end + 255) / 256 * 256;
}

size_t gdn_prefill_fused_workspace_bytes(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens) {
  if (check_config(cfg) != GDN_OK || n_seqs < 0 || n_tokens < 0) return 0;
  if (n_tokens == 0) return 0;
  return fused_ready_offset(cfg, n_seqs, n_tokens) +
         static_cast<size_t>(gdn::max_chunks(n_seqs, n_tokens)) * cfg->n_v_heads * gdn::kReadyStride * sizeof(uint32_t);
}

gdn_status gdn_prefill_fused_ckpt(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens,
                                  const int32_t *cu_seqlens, const void *qkv, const void *beta_logit,
                                  const void *alpha_logit, const void *z, const float *conv_w,
                                  const float *dt_bias, const float *A_log, const float *norm_w,
                                  const void *conv_state_in, void *conv_state_out, const float *S_in, float *S_out,
                                  void *y, int32_t ckpt_every, int32_t ckpt_cap, float *S_ckpt, void *conv_ckpt,
                                  void *workspace, size_t workspace_bytes, gdn_stream_t stream) {
  const gdn_status cs = check_config(cfg);
  if (cs != GDN_OK) return cs;
  if (n_seqs < 0 || n_tokens < 0) return GDN_E_INVALID_ARG;
  if (n_seqs == 0) return n_tokens == 0 ? GDN_OK : GDN_E_INVALID_ARG;
  if (ckpt_every < 0 || ckpt_cap < 0 || ckpt_every % gdn::kChunk != 0) return GDN_E_INVALID_ARG;
  const bool ckpt = ckpt_every > 0 && ckpt_cap > 0;
  if (ckpt && !S_ckpt) return GDN_E_INVALID_ARG;
  if (!cu_seqlens || !conv_w || !dt_bias || !A_log || !norm_w || !conv_state_in || !conv_state_out || !S_in ||
      !S_out)
    return GDN_E_INVALID_ARG;
  if (n_tokens > 0 && (!qkv || !beta_logit || !alpha_logit || !z || !y)) return GDN_E_INVALID_ARG;
  // The chunk kernels read qkv and the conv state 16 bytes at a time; the
  // norm reads o and z and writes y 16 bytes at a time.
  const Align al[] = {{qkv, 16}, {conv_state_in, 16}, {conv_state_out, 16}, {conv_w, 16},
                      {z, 16}, {y, 16}, {norm_w, 16}};
  if (!all_aligned(al)) return GDN_E_INVALID_ARG;
  const int Hqk = cfg->n_qk_heads, Hv = cfg->n_v_heads;
  const size_t need = gdn_prefill_fused_workspace_bytes(cfg, n_seqs, n_tokens);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return GDN_E_WORKSPACE;
  const int64_t chunks = gdn::max_chunks(n_seqs, n_tokens);
  const size_t T = static_cast<size_t>(n_tokens), as = act_size(cfg);
  const size_t C = static_cast<size_t>(kHeadDim) * (2 * Hqk + Hv);
  if (chunks > kMaxGrid || Hqk > 65535 || static_cast<int64_t>(n_seqs) * Hv * (kHeadDim / 32) > kMaxGrid ||
      static_cast<int64_t>(n_seqs) * static_cast<int64_t>((C / 2 + 255) / 256) > kMaxGrid)
    return GDN_E_UNSUPPORTED;
  const size_t st = static_cast<size_t>(n_seqs) * (gdn::kConvK - 1) * C * as;
  const size_t sb = static_cast<size_t>(n_seqs) * Hv * kHeadDim * kHeadDim * 4;
  const size_t yb = T * Hv * kHeadDim * as;
  const Range outs[] = {{y, yb}, {workspace, need}};
  const Range ins[] = {{qkv, T * C * as}, {beta_logit, T * Hv * as}, {alpha_logit, T * Hv * as}, {z, yb},
                       {conv_w, C * 4 * 4}, {dt_bias, Hv * 4u}, {A_log, Hv * 4u}, {norm_w, kHeadDim * 4u},
                       {cu_seqlens, (n_seqs + 1u) * 4u}, {conv_state_in, st}, {conv_state_out, st},
                       {S_in, sb}, {S_out, sb}};
  if (any_overlap(outs, ins)) return GDN_E_INVALID_ARG;
  // Each state may be updated in place, but must not partly overlap or
  // overlap anything else.
  if (conv_state_in != conv_state_out && overlap(conv_state_in, st, conv_state_out, st)) return GDN_E_INVALID_ARG;
  if (S_in != S_out && overlap(S_in, sb, S_out, sb)) return GDN_E_INVALID_ARG;
  for (size_t i = 0; i < 9; ++i)
    if (overlap(ins[i].p, ins[i].n, conv_state_out, st) || overlap(ins[i].p, ins[i].n, S_out, sb))
      return GDN_E_INVALID_ARG;
  if (overlap(conv_state_out, st, S_out, sb) || overlap(conv_state_in, st, S_out, sb) ||
      overlap(conv_state_out, st, S_in, sb))
    return GDN_E_INVALID_ARG;
  if (ckpt) {
    // The checkpoint planes overlap nothing else.
    const size_t cb = static_cast<size_t>(n_seqs) * ckpt_cap * Hv * kHeadDim * kHeadDim * 4;
    const size_t ccb = conv_ckpt ? static_cast<size_t>(n_seqs) * ckpt_cap * (gdn::kConvK - 1) * C * as : 0;
    if (conv_ckpt && !aligned(conv_ckpt, 2 * as)) return GDN_E_INVALID_ARG;
    for (const Range &r : ins)
      if (overlap(r.p, r.n, S_ckpt, cb) || overlap(r.p, r.n, conv_ckpt, ccb)) return GDN_E_INVALID_ARG;
    if (overlap(y, yb, S_ckpt, cb) || overlap(workspace, need, S_ckpt, cb) || overlap(y, yb, conv_ckpt, ccb) ||
        overlap(workspace, need, conv_ckpt, ccb) || overlap(S_ckpt, cb, conv_ckpt, ccb))
      return GDN_E_INVALID_ARG;
    if (static_cast<int64_t>(n_seqs) * ckpt_cap > kMaxGrid) return GDN_E_UNSUPPORTED;
  }

  const hipStream_t hs = static_cast<hipStream_t>(stream);
  void *o = n_tokens > 0 ? static_cast<uint8_t *>(workspace) + fused_o_offset(cfg, n_seqs, n_tokens) : nullptr;
  gdn::PrefillParams p = {};
  p.cu = cu_seqlens;
  p.n_seqs = n_seqs;
  p.n_tokens = n_tokens;
  p.n_qk = Hqk;
  p.n_v = Hv;
  p.S_in = S_in;
  p.S_out = S_out;
  p.o = o;
  p.ws = workspace;
  p.ws_bytes = workspace_bytes;
  p.qkv = n_tokens > 0 ? qkv : conv_state_in;   // non-null selects the fused kernels
  p.bl = beta_logit;
  p.al = alpha_logit;
  p.st_in = conv_state_in;
  p.conv_w = conv_w;
  p.dt_bias = dt_bias;
  p.A_log = A_log;
  p.l2_eps = cfg->l2_eps;
  p.l2_mode = cfg->l2_mode;
  p.S_ckpt = ckpt ? S_ckpt : nullptr;
  p.ckpt_chunks = ckpt ? ckpt_every / gdn::kChunk : 0;
  p.ckpt_cap = ckpt ? ckpt_cap : 0;
  // The gated RMSNorm and the new conv states are formed inside the
  // sequential kernel's launch when that leaves CUs idle, else by a launch of
  // their own after it.
  p.fold_blocks = n_tokens > 0 ? gdn::prefill_fold_blocks(n_seqs, Hv) : 0;
  if (p.fold_blocks > 0) {
    p.ready = reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(workspace) +
                                           fused_ready_offset(cfg, n_seqs, n_tokens));
    p.z = z;
    p.norm_w = norm_w;
    p.y = y;
    p.norm_eps = cfg->norm_eps;
    p.st_out = conv_state_out;
  }
  hipError_t e = hipSuccess;
  if (ckpt && conv_ckpt && n_tokens > 0) {
    // Conv-state planes, first: they read the old conv state, which the
    // launches below may update in place.
    gdn::ConvCkptParams cp;
    cp.cu = cu_seqlens;
    cp.n_seqs = n_seqs;
    cp.n_tokens = n_tokens;
    cp.n_qk = Hqk;
    cp.n_v = Hv;
    cp.every = ckpt_every;
    cp.cap = ckpt_cap;
    cp.qkv = qkv;
    cp.st_in = conv_state_in;
    cp.ckpt = conv_ckpt;
    e = gdn::launch_conv_ckpt(cp, cfg->act_dtype, hs);
  }
  if (e == hipSuccess) e = gdn::launch_prefill(p, cfg->act_dtype, hs);
  if (e == hipSuccess && p.fold_blocks == 0) {
    // The norm, and the new conv states: last, since the kernels above read
    // the old conv state (in-place safe).
    gdn::NormParams np;
    np.n_rows = static_cast<int64_t>(n_tokens) * Hv;
    np.o = o;
    np.z = z;
    np.w = norm_w;
    np.y = y;
    np.eps = cfg->norm_eps;
    gdn::ConvStateParams cp;
    cp.cu = cu_seqlens;
    cp.n_seqs = n_seqs;
    cp.n_tokens = n_tokens;
    cp.C = static_cast<int>(C);
    cp.qkv = qkv;
    cp.st_in = conv_state_in;
    cp.st_out = conv_state_out;
    e = gdn::launch_norm_conv_state(np, cp, cfg->act_dtype, hs);
  }
  return launched(e);
}

gdn_status gdn_prefill_fused(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens, const int32_t *cu_seqlens,
                             const void *qkv, const void *beta_logit, const void *alpha_logit, const void *z,
                             const float *conv_w, const float *dt_bias, const float *A_log, const float *norm_w,
                             const void *conv_state_in, void *conv_state_out, const float *S_in, float *S_out,
                             void *y, void *workspace, size_t workspace_bytes, gdn_stream_t stream) {
  return gdn_prefill_fused_ckpt(cfg, n_seqs, n_tokens, cu_seqlens, qkv, beta_logit, alpha_logit, z, conv_w, dt_bias,
                                A_log, norm_w, conv_state_in, conv_state_out, S_in, S_out, y, 0, 0, nullptr,
                                nullptr, workspace, workspace_bytes, stream);
}

gdn_status gdn_conv_state_ckpt(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens, const int32_t *cu_seqlens,
                               const void *qkv, const void *conv_state_in, int32_t ckpt_every, int32_t ckpt_cap,
                               void *conv_ckpt, gdn_stream_t stream) {
  const gdn_status cs = check_config(cfg);
  if (cs != GDN_OK) return cs;
  if (n_seqs < 0 || n_tokens < 0 || ckpt_every < 1 || ckpt_cap < 0) return GDN_E_INVALID_ARG;
  if (n_seqs == 0 || ckpt_cap == 0) return GDN_OK;
  if (!cu_seqlens || !conv_state_in || !conv_ckpt || (n_tokens > 0 && !qkv)) return GDN_E_INVALID_ARG;
  if (static_cast<int64_t>(n_seqs) * ckpt_cap > kMaxGrid) return GDN_E_UNSUPPORTED;
  const int Hqk = cfg->n_qk_heads, Hv = cfg->n_v_heads;
  const size_t as = act_size(cfg), C = static_cast<size_t>(kHeadDim) * (2 * Hqk + Hv);
  const Align al[] = {{qkv, 2 * as}, {conv_state_in, 2 * as}, {conv_ckpt, 2 * as}};
  if (!all_aligned(al)) return GDN_E_INVALID_ARG;
  const size_t st = static_cast<size_t>(n_seqs) * (gdn::kConvK - 1) * C * as;
  const Range outs[] = {{conv_ckpt, static_cast<size_t>(n_seqs) * ckpt_cap * (gdn::kConvK - 1) * C * as}};
  const Range ins[] = {{qkv, static_cast<size_t>(n_tokens) * C * as}, {conv_state_in, st},
                       {cu_seqlens, (n_seqs + 1u) * 4u}};
  if (any_overlap(outs, ins)) return GDN_E_INVALID_ARG;
  gdn::ConvCkptParams p;
  p.cu = cu_seqlens;
  p.n_seqs = n_seqs;
  p.n_tokens = n_tokens;
  p.n_qk = Hqk;
  p.n_v = Hv;
  p.every = ckpt_every;
  p.cap = ckpt_cap;
  p.qkv = qkv;
  p.st_in = conv_state_in;
  p.ckpt = conv_ckpt;
  return launched(gdn::launch_conv_ckpt(p, cfg->act_dtype, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_state_check(const float *S, int64_t n_values, int32_t *stats, gdn_stream_t stream) {
  if (n_values < 0 || !stats || (n_values > 0 && !S)) return GDN_E_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(S) % 16 != 0 || reinterpret_cast<uintptr_t>(stats) % 4 != 0)
    return GDN_E_INVALID_ARG;
  if (overlap(S, static_cast<size_t>(n_values) * 4, stats, 8)) return GDN_E_INVALID_ARG;
  return launched(gdn::launch_state_check(S, n_values, stats, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_decode_step(const gdn_config *cfg, int32_t n_seqs, const float *q, const float *k,
                           const float *v, const float *beta, const float *g, const float *S_in,
                           float *S_out, void *o, gdn_stream_t stream) {
  const gdn_status cs = check_config(cfg);
  if (cs != GDN_OK) return cs;
  if (n_seqs < 0) return GDN_E_INVALID_ARG;
  if (n_seqs == 0) return GDN_OK;
  if (!q || !k || !v || !beta || !g || !S_in || !S_out || !o) return GDN_E_INVALID_ARG;
  // State, q, k, v read 4 floats at a time; o written 4 values at a time.
  const Align al[] = {{S_in, 16}, {S_out, 16}, {q, 16}, {k, 16}, {v, 16}, {o, 4 * act_size(cfg)}};
  if (!all_aligned(al)) return GDN_E_INVALID_ARG;
  const int Hqk = cfg->n_qk_heads, Hv = cfg->n_v_heads;
  if (static_cast<int64_t>(n_seqs) * Hv * (kHeadDim / 32) > kMaxGrid) return GDN_E_UNSUPPORTED;
  const size_t N = static_cast<size_t>(n_seqs);
  const size_t sb = N * Hv * kHeadDim * kHeadDim * 4;
  const Range outs[] = {{o, N * Hv * kHeadDim * act_size(cfg)}};
  const Range ins[] = {{q, N * Hqk * kHeadDim * 4}, {k, N * Hqk * kHeadDim * 4}, {v, N * Hv * kHeadDim * 4},
                       {beta, N * Hv * 4}, {g, N * Hv * 4}, {S_in, sb}, {S_out, sb}};
  if (any_overlap(outs, ins)) return GDN_E_INVALID_ARG;
  if (S_in != S_out && overlap(S_in, sb, S_out, sb)) return GDN_E_INVALID_ARG;
  for (size_t i = 0; i < 5; ++i)
    if (overlap(ins[i].p, ins[i].n, S_out, sb)) return GDN_E_INVALID_ARG;

  gdn::DecodeParams p;
  p.n_seqs = n_seqs;
  p.n_qk = Hqk;
  p.n_v = Hv;
  p.q = q;
  p.k = k;
  p.v = v;
  p.beta = beta;
  p.g = g;
  p.S_in = S_in;
  p.S_out = S_out;
  p.o = o;
  return launched(gdn::launch_decode(p, cfg->act_dtype, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Shared checks of the two projections: bf16 only, K (the contraction length)
// a positive multiple of 64, operands 16-byte aligned.
gdn_status check_proj(const gdn_config *cfg, int32_t n_tokens, int32_t hidden) {
  const gdn_status cs = check_config(cfg);
  if (cs != GDN_OK) return cs;
  if (n_tokens < 0 || hidden < 1) return GDN_E_INVALID_ARG;
  if (cfg->act_dtype != GDN_BF16 || hidden % 64 != 0) return GDN_E_UNSUPPORTED;
  return GDN_OK;
}

gdn_status launch_proj(const gdn::GemmParams &p, gdn_stream_t stream) {
  // Tiles of 256 rows by at least 128 columns; the grid is far below its limit
  // for any int32 sizes, but the row index arithmetic needs M * K in int64.
  return launched(gdn::launch_gemm(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

gdn_status gdn_in_proj(const gdn_config *cfg, int32_t n_tokens, int32_t hidden, const void *x, const void *w_qkv,
                       const void *w_gate, const void *w_beta, const void *w_alpha, void *qkv, void *z,
                       void *beta_logit, void *alpha_logit, gdn_stream_t stream) {
  const gdn_status cs = check_proj(cfg, n_tokens, hidden);
  if (cs != GDN_OK) return cs;
  if (n_tokens == 0) return GDN_OK;
  if (!x || !w_qkv || !w_gate || !w_beta || !w_alpha || !qkv || !z || !beta_logit || !alpha_logit)
    return GDN_E_INVALID_ARG;
  const void *ops[] = {x, w_qkv, w_gate, w_beta, w_alpha};
  for (const void *o : ops)
    if (!aligned(o, 16)) return GDN_E_INVALID_ARG;
  const void *res[] = {qkv, z, beta_logit, alpha_logit};
  for (const void *o : res)
    if (!aligned(o, 2)) return GDN_E_INVALID_ARG;
  const int Hqk = cfg->n_qk_heads, Hv = cfg->n_v_heads;
  const int64_t C = static_cast<int64_t>(kHeadDim) * (2 * Hqk + Hv), Z = static_cast<int64_t>(Hv) * kHeadDim;
  const int64_t N = C + Z + 2 * Hv;
  if (N > kMaxGrid) return GDN_E_UNSUPPORTED;
  const size_t T = static_cast<size_t>(n_tokens), H = static_cast<size_t>(hidden);
  const Range outs[] = {{qkv, T * C * 2}, {z, T * Z * 2}, {beta_logit, T * Hv * 2}, {alpha_logit, T * Hv * 2}};
  const Range ins[] = {{x, T * H * 2}, {w_qkv, C * H * 2}, {w_gate, Z * H * 2}, {w_beta, Hv * H * 2},
                       {w_alpha, Hv * H * 2}};
  if (any_overlap(outs, ins)) return GDN_E_INVALID_ARG;

  gdn::GemmParams p;
  p.M = n_tokens;
  p.N = static_cast<int>(N);
  p.K = hidden;
  p.x = static_cast<const uint16_t *>(x);
  p.n_seg = 4;
  const int64_t start[4] = {0, C, C + Z, C + Z + Hv};
  const void *w[4] = {w_qkv, w_gate, w_beta, w_alpha};
  void *out[4] = {qkv, z, beta_logit, alpha_logit};
  const int64_t ld[4] = {C, Z, Hv, Hv};
  for (int s = 0; s < 4; ++s) {
    p.start[s] = static_cast<int>(start[s]);
    p.w[s] = static_cast<const uint16_t *>(w[s]);
    p.out[s] = static_cast<uint16_t *>(out[s]);
    p.ld[s] = ld[s];
  }
  return launch_proj(p, stream);
}

gdn_status gdn_out_proj(const gdn_config *cfg, int32_t n_tokens, int32_t hidden, const void *y, const void *w_out,
                        void *out, gdn_stream_t stream) {
  const gdn_status cs = check_config(cfg);
  if (cs != GDN_OK) return cs;
  if (n_tokens < 0 || hidden < 1) return GDN_E_INVALID_ARG;
  if (cfg->act_dtype != GDN_BF16) return GDN_E_UNSUPPORTED;
  if (n_tokens == 0) return GDN_OK;
  if (!y || !w_out || !out) return GDN_E_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(w_out, 16) || !aligned(out, 2)) return GDN_E_INVALID_ARG;
  const int64_t Kd = static_cast<int64_t>(cfg->n_v_heads) * kHeadDim;
  if (Kd > kMaxGrid) return GDN_E_UNSUPPORTED;
  const size_t T = static_cast<size_t>(n_tokens), H = static_cast<size_t>(hidden);
  const Range outs[] = {{out, T * H * 2}};
  const Range ins[] = {{y, T * Kd * 2}, {w_out, H * Kd * 2}};
  if (any_overlap(outs, ins)) return GDN_E_INVALID_ARG;

  gdn::GemmParams p = {};
  p.M = n_tokens;
  p.N = hidden;
  p.K = static_cast<int>(Kd);
  p.x = static_cast<const uint16_t *>(y);
  p.n_seg = 1;
  p.w[0] = static_cast<const uint16_t *>(w_out);
  p.out[0] = static_cast<uint16_t *>(out);
  p.ld[0] = hidden;
  return launch_proj(p, stream);
}

}  // extern "C"

namespace {

// gdn_decode_fused (K = 1) and gdn_decode_verify: K tokens per sequence in one
// launch, the state and conv state after each token to its snapshot plane.
gdn_status decode_tokens(const gdn_config *cfg, int32_t n_seqs, int32_t K, const void *qkv,
                         const void *beta_logit, const void *alpha_logit, const void *z, const float *conv_w,
                         const float *dt_bias, const float *A_log, const float *norm_w,
                         const void *conv_state_in, void *conv_snap, const float *S_in, float *S_snap,
                         void *y, gdn_stream_t stream) {
  const gdn_status cs = check_config(cfg);
  if (cs != GDN_OK) return cs;
  if (n_seqs < 0 || K < 0) return GDN_E_INVALID_ARG;
  if (n_seqs == 0 || K == 0) return GDN_OK;
  if (!qkv || !beta_logit || !alpha_logit || !z || !conv_w || !dt_bias || !A_log || !norm_w ||
      !conv_state_in || !conv_snap || !S_in || !S_snap || !y)
    return GDN_E_INVALID_ARG;
  {
    // State, norm weights and conv taps 16 bytes at a time; z and y four
    // values, qkv and the conv states two values at a time.
    const size_t as = act_size(cfg);
    const Align al[] = {{S_in, 16}, {S_snap, 16}, {norm_w, 16}, {conv_w, 16}, {z, 4 * as}, {y, 4 * as},
                        {qkv, 2 * as}, {conv_state_in, 2 * as}, {conv_snap, 2 * as}};
    if (!all_aligned(al)) return GDN_E_INVALID_ARG;
  }
  const int Hqk = cfg->n_qk_heads, Hv = cfg->n_v_heads;
  if (static_cast<int64_t>(n_seqs) * Hv > kMaxGrid) return GDN_E_UNSUPPORTED;
  const size_t N = static_cast<size_t>(n_seqs), NK = N * static_cast<size_t>(K), as = act_size(cfg);
  const size_t C = static_cast<size_t>(kHeadDim) * (2 * Hqk + Hv);
  const size_t sb = N * Hv * kHeadDim * kHeadDim * 4, snap = NK * Hv * kHeadDim * kHeadDim * 4;
  const size_t st = N * (gdn::kConvK - 1) * C * as, cst = NK * (gdn::kConvK - 1) * C * as;
  const Range outs[] = {{y, NK * Hv * kHeadDim * as}, {conv_snap, cst}};
  const Range ins[] = {{qkv, NK * C * as}, {beta_logit, NK * Hv * as}, {alpha_logit, NK * Hv * as},
                       {z, NK * Hv * kHeadDim * as}, {conv_w, C * 4 * 4}, {dt_bias, Hv * 4u},
                       {A_log, Hv * 4u}, {norm_w, kHeadDim * 4u}, {conv_state_in, st}, {S_in, sb}, {S_snap, snap}};
  if (any_overlap(outs, ins)) return GDN_E_INVALID_ARG;
  // A single step may update S in place; K > 1 needs the snapshot planes apart from S_in.
  if (overlap(S_in, sb, S_snap, snap) && !(K == 1 && S_in == S_snap)) return GDN_E_INVALID_ARG;
  for (size_t i = 0; i < 9; ++i)
    if (overlap(ins[i].p, ins[i].n, S_snap, snap)) return GDN_E_INVALID_ARG;

  gdn::FusedDecodeParams p;
  p.n_seqs = n_seqs;
  p.n_tok = K;
  p.n_qk = Hqk;
  p.n_v = Hv;
  p.qkv = qkv;
  p.b = beta_logit;
  p.a = alpha_logit;
  p.z = z;
  p.conv_w = conv_w;
  p.dt_bias = dt_bias;
  p.A_log = A_log;
  p.norm_w = norm_w;
  p.st_in = conv_state_in;
  p.st_out = conv_snap;
  p.S_in = S_in;
  p.S_out = S_snap;
  p.y = y;
  p.l2_eps = cfg->l2_eps;
  p.l2_mode = cfg->l2_mode;
  p.norm_eps = cfg->norm_eps;
  return launched(gdn::launch_decode_fused(p, cfg->act_dtype, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

gdn_status gdn_decode_fused(const gdn_config *cfg, int32_t n_seqs, const void *qkv, const void *beta_logit,
                            const void *alpha_logit, const void *z, const float *conv_w, const float *dt_bias,
                            const float *A_log, const float *norm_w, const void *conv_state_in,
                            void *conv_state_out, const float *S_in, float *S_out, void *y,
                            gdn_stream_t stream) {
  return decode_tokens(cfg, n_seqs, 1, qkv, beta_logit, alpha_logit, z, conv_w, dt_bias, A_log, norm_w,
                       conv_state_in, conv_state_out, S_in, S_out, y, stream);
}

gdn_status gdn_decode_verify(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens, const void *qkv,
                             const void *beta_logit, const void *alpha_logit, const void *z,
                             const float *conv_w, const float *dt_bias, const float *A_log,
                             const float *norm_w, const void *conv_state_in, void *conv_snap,
                             const float *S_in, float *S_snap, void *y, gdn_stream_t stream) {
  return decode_tokens(cfg, n_seqs, n_tokens, qkv, beta_logit, alpha_logit, z, conv_w, dt_bias, A_log, norm_w,
                       conv_state_in, conv_snap, S_in, S_snap, y, stream);
}

gdn_status gdn_gated_rmsnorm(const gdn_config *cfg, int64_t n_rows, const void *o, const void *z,
                             const float *norm_w, void *y, gdn_stream_t stream) {
  const gdn_status cs = check_config(cfg);
  if (cs != GDN_OK) return cs;
  if (n_rows < 0) return GDN_E_INVALID_ARG;
  if (n_rows == 0) return GDN_OK;
  if (!o || !z || !norm_w || !y) return GDN_E_INVALID_ARG;
  // Eight values of o, z, y and four weights per access: 16 bytes.
  const Align al[] = {{o, 16}, {z, 16}, {y, 16}, {norm_w, 16}};
  if (!all_aligned(al)) return GDN_E_INVALID_ARG;
  if ((n_rows + 15) / 16 > kMaxGrid) return GDN_E_UNSUPPORTED;
  const size_t bytes = static_cast<size_t>(n_rows) * kHeadDim * act_size(cfg);
  // y may be o (in place); nothing else may overlap y.
  if (y != o && overlap(y, bytes, o, bytes)) return GDN_E_INVALID_ARG;
  if (overlap(y, bytes, z, bytes) || overlap(y, bytes, norm_w, kHeadDim * 4)) return GDN_E_INVALID_ARG;
  gdn::NormParams p;
  p.n_rows = n_rows;
  p.o = o;
  p.z = z;
  p.w = norm_w;
  p.y = y;
  p.eps = cfg->norm_eps;
  return launched(gdn::launch_norm(p, cfg->act_dtype, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// gdn_prefill_fused_static: gdn_prefill_fused with its workspace in a
// file-scope device array instead of a caller buffer, for callers that cannot
// allocate. Each device that runs it holds its own copy of the array from the
// time the library's code is loaded there until the process ends. In host code
// `scratch` is only a stand-in: its device address, which differs per device,
// is looked up once per device with hipGetSymbolAddress (with that device
// current) and kept in scratch_ptr, and only that address is ever handed to a
// kernel.
namespace {

constexpr size_t kStaticScratchBytes = static_cast<size_t>(GDN_STATIC_SCRATCH_BYTES);
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (looked up on first use).
gdn_status static_scratch(hipStream_t stream, void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GDN_E_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return GDN_E_HIP;
    if (sdev != dev) return GDN_E_INVALID_ARG;   // the stream must belong to the current device
  }
  if (dev < 0 || dev >= kMaxDevices) return GDN_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN_E_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_fused_static(const gdn_config *cfg, int32_t n_seqs, int32_t n_tokens,
                                    const int32_t *cu_seqlens, const void *qkv, const void *beta_logit,
                                    const void *alpha_logit, const void *z, const float *conv_w,
                                    const float *dt_bias, const float *A_log, const float *norm_w,
                                    const void *conv_state_in, void *conv_state_out, const float *S_in,
                                    float *S_out, void *y, gdn_stream_t stream) {
  const gdn_status cs = check_config(cfg);
  if (cs != GDN_OK) return cs;
  if (n_seqs < 0 || n_tokens < 0) return GDN_E_INVALID_ARG;
  const size_t need = gdn_prefill_fused_workspace_bytes(cfg, n_seqs, n_tokens);
  if (need > kStaticScratchBytes) return GDN_E_TOO_LARGE;
  void *ws = nullptr;
  if (need > 0) {
    const gdn_status ss = static_scratch(static_cast<hipStream_t>(stream), &ws);
    if (ss != GDN_OK) return ss;
  }
  return gdn_prefill_fused(cfg, n_seqs, n_tokens, cu_seqlens, qkv, beta_logit, alpha_logit, z, conv_w, dt_bias,
                           A_log, norm_w, conv_state_in, conv_state_out, S_in, S_out, y, ws,
                           need > 0 ? kStaticScratchBytes : 0, stream);
}

}  // extern "C"
