/*
 * gdn_oracle.c -- plain fp64 CPU oracle of the gated DeltaNet token mixer.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg may build, load or call this file. The HIP
 * library never links it, and it includes nothing from the HIP library.
 *
 * Source of the method: the xwen CLAUDE.md page, section "Architecture cheat
 * sheet", paragraph on the gated DeltaNet layer, with the RMSNorm epsilon from
 * the paragraph shared by both models in that section, and the GGUF facts
 * (norm weights used as stored, ssm_a = -exp(A_log), tiled V-head order) from
 * the section "GGUF facts that differ from the HF checkpoint".
 *
 * Everything is computed token by token in fp64, in the order the page lists
 * the steps, with no blocking, fusion or reordering. Readings of points the
 * page leaves open are marked "Reading:".
 *
 * Layouts (row-major, last index fastest):
 *   qkv     [T][C]           C = d*(2*Hqk + Hv), q block | k block | v block,
 *                            each head-major with d contiguous values per head
 *   conv_w  [C][4]           tap j meets the row 3-j tokens before the current one
 *   conv_in / conv_out [N][3][C]   the 3 raw (pre-conv) rows preceding the
 *                            sequence, oldest first
 *   q, k    [T][Hqk][d]      L2-normalised
 *   v       [T][Hv][d]
 *   beta, g [T][Hv]
 *   S_in / S_out [N][Hv][d][d]  S[i][c]: i = key index, c = value index
 *   o       [T][Hv][d]       readout before the gated norm
 *   z, y    [T][Hv][d]
 * Sequences are packed: sequence n owns tokens cu[n] .. cu[n+1]-1.
 */
#include <math.h>
#include <stddef.h>
#include <string.h>

/* The conv kernel size the page fixes for this layer. */
#define GDNO_CONV_K 4

/* sigmoid(x) = 1 / (1 + e^-x). */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* softplus(x) = log(1 + e^x), evaluated without overflow as
 * max(x, 0) + log1p(e^-|x|).  Reading: the page names softplus without
 * giving its numerics; this is the same function evaluated stably. */
static double softplus(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

/* SiLU(x) = x * sigmoid(x). */
static double silu(double x) { return x * sigmoid(x); }

/*
 * Conv, SiLU, split, L2 clamp-norm and gates for every token.
 *
 * Conv: depthwise over all C fused channels, kernel 4, causal, no bias.
 * For sequence n let X be its 3 conv-state rows followed by its L tokens'
 * qkv rows (L+3 rows). The conv output of local token t is
 *     y[c] = sum_{j=0..3} conv_w[c][j] * X[t + j][c]
 * so tap 3 meets the current token and tap 0 the token three back.
 * Reading: the page states "kernel 4, causal" only; this tap order is the
 * plain causal cross-correlation with 3 rows of left context.
 * The new conv state is the last 3 rows of X (raw inputs, copied).
 * Reading: the page calls the conv state the last 3 columns of the fused qkv
 * stream; they are the raw rows the next call's first outputs need.
 *
 * SiLU runs over all C channels (q and k too) before the split.
 * q_h = y[d*h ..], k_h = y[d*Hqk + d*h ..], v_j = y[2*d*Hqk + d*j ..].
 * q and k are normalised in the clamp form x / max(||x||_2, l2_eps)
 * (l2_mode 0, the page's canonical form), or, with l2_mode 1, in the form
 * x / sqrt(sum x^2 + l2_eps) that the page notes for the HF checkpoint.
 * beta = sigmoid(b); g = -exp(A_log) * softplus(a + dt_bias).
 */
void gdno_conv_gate_prep(int n_seqs, const int *cu, int Hqk, int Hv, int d,
                         const double *qkv, const double *b, const double *a,
                         const double *conv_w, const double *dt_bias, const double *A_log,
                         const double *conv_in, double l2_eps, int l2_mode,
                         double *conv_out, double *q, double *k, double *v,
                         double *beta, double *g)
{
    const int C = d * (2 * Hqk + Hv);
    const int KS = GDNO_CONV_K - 1;   /* 3 rows of state */
    for (int n = 0; n < n_seqs; ++n) {
        const int t0 = cu[n], L = cu[n + 1] - cu[n];
        const double *st = conv_in + (size_t)n * KS * C;
        for (int t = 0; t < L; ++t) {
            const size_t tok = (size_t)(t0 + t);
            for (int h = 0; h < Hqk; ++h) {
                /* q and k of head h: conv + silu, then the clamp-form L2 norm. */
                for (int part = 0; part < 2; ++part) {
                    const int c0 = part * d * Hqk + h * d;
                    double *dst = (part == 0 ? q : k) + (tok * Hqk + h) * d;
                    double ss = 0.0;
                    for (int i = 0; i < d; ++i) {
                        const int c = c0 + i;
                        double acc = 0.0;
                        for (int j = 0; j < GDNO_CONV_K; ++j) {
                            const int r = t + j;           /* row of X */
                            const double x = r < KS ? st[(size_t)r * C + c]
                                                    : qkv[(size_t)(t0 + r - KS) * C + c];
                            acc += conv_w[(size_t)c * GDNO_CONV_K + j] * x;
                        }
                        dst[i] = silu(acc);
                        ss += dst[i] * dst[i];
                    }
                    const double nrm = sqrt(ss);
                    const double den = nrm > l2_eps ? nrm : l2_eps;
                    const double den_hf = sqrt(ss + l2_eps);
                    for (int i = 0; i < d; ++i) dst[i] /= (l2_mode == 1 ? den_hf : den);
                }
            }
            for (int jh = 0; jh < Hv; ++jh) {
                const int c0 = 2 * d * Hqk + jh * d;
                double *dst = v + (tok * Hv + jh) * d;
                for (int i = 0; i < d; ++i) {
                    const int c = c0 + i;
                    double acc = 0.0;
                    for (int j = 0; j < GDNO_CONV_K; ++j) {
                        const int r = t + j;
                        const double x = r < KS ? st[(size_t)r * C + c]
                                                : qkv[(size_t)(t0 + r - KS) * C + c];
                        acc += conv_w[(size_t)c * GDNO_CONV_K + j] * x;
                    }
                    dst[i] = silu(acc);
                }
                const size_t e = tok * Hv + jh;
                beta[e] = sigmoid(b[e]);
                g[e] = -exp(A_log[jh]) * softplus(a[e] + dt_bias[jh]);
            }
        }
        /* New conv state: rows L, L+1, L+2 of X. */
        for (int r = 0; r < KS; ++r) {
            const int src = L + r;
            for (int c = 0; c < C; ++c) {
                conv_out[((size_t)n * KS + r) * C + c] =
                    src < KS ? st[(size_t)src * C + c] : qkv[(size_t)(t0 + src - KS) * C + c];
            }
        }
    }
}

/*
 * The delta rule in its recurrent form, one token at a time, per sequence
 * and per V-head j, with S the d x d fp64 state (S[i][c]):
 *     S <- exp(g) * S
 *     u[c]  = sum_i S[i][c] * k[i]            (S . k)
 *     dl[c] = beta * (v[c] - u[c])
 *     S[i][c] += k[i] * dl[c]                 (k outer d)
 *     o[c]  = (1/sqrt(d)) * sum_i S[i][c] * q[i]   (read from the updated S)
 * V-head j uses the q/k of K-head j mod Hqk (tiled repeat, not interleave).
 * Reading: the page writes the products as S.k and k (x) d without naming
 * which axis of S is the key axis; S[i][c] with i the key index is the
 * orientation under which both products are well formed.
 * Reading: the readout scale is 1/sqrt(d); the page fixes d = 128.
 *
 * head_sel (nullable, length Hv): when given, only V-heads with a nonzero
 * flag are computed; o and S_out of the others are left untouched.
 * S_in and S_out may be the same buffer.
 */
void gdno_delta_rule(int n_seqs, const int *cu, int Hqk, int Hv, int d,
                     const double *q, const double *k, const double *v,
                     const double *beta, const double *g,
                     const double *S_in, double *S_out, double *o,
                     const int *head_sel, double *work /* d*d + 2*d */)
{
    const double scale = 1.0 / sqrt((double)d);
    double *S = work, *u = work + (size_t)d * d, *dl = u + d;
    for (int n = 0; n < n_seqs; ++n) {
        const int t0 = cu[n], L = cu[n + 1] - cu[n];
        for (int j = 0; j < Hv; ++j) {
            if (head_sel && !head_sel[j]) continue;
            const int hk = j % Hqk;
            const size_t sb = ((size_t)n * Hv + j) * d * d;
            memcpy(S, S_in + sb, sizeof(double) * (size_t)d * d);
            for (int t = 0; t < L; ++t) {
                const size_t tok = (size_t)(t0 + t);
                const double *kv = k + (tok * Hqk + hk) * d;
                const double *qv = q + (tok * Hqk + hk) * d;
                const double *vv = v + (tok * Hv + j) * d;
                const double bt = beta[tok * Hv + j];
                const double decay = exp(g[tok * Hv + j]);
                for (size_t e = 0; e < (size_t)d * d; ++e) S[e] *= decay;
                for (int c = 0; c < d; ++c) {
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i) acc += S[(size_t)i * d + c] * kv[i];
                    u[c] = acc;
                }
                for (int c = 0; c < d; ++c) dl[c] = bt * (vv[c] - u[c]);
                for (int i = 0; i < d; ++i)
                    for (int c = 0; c < d; ++c) S[(size_t)i * d + c] += kv[i] * dl[c];
                double *ov = o + (tok * Hv + j) * d;
                for (int c = 0; c < d; ++c) {
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i) acc += S[(size_t)i * d + c] * qv[i];
                    ov[c] = scale * acc;
                }
            }
            memcpy(S_out + sb, S, sizeof(double) * (size_t)d * d);
        }
    }
}

/*
 * Gated RMSNorm per (token, V-head) row of d values:
 *     r = sqrt(mean_c o[c]^2 + eps)
 *     y[c] = (o[c] / r) * w[c] * silu(z[c])
 * The weight w[d] is shared by all heads and used as stored (no +1), and the
 * norm weight multiplies before the silu(z) gate.
 */
void gdno_gated_rmsnorm(long n_rows, int d, const double *o, const double *z,
                        const double *w, double eps, double *y)
{
    for (long r = 0; r < n_rows; ++r) {
        const double *orow = o + (size_t)r * d, *zrow = z + (size_t)r * d;
        double ss = 0.0;
        for (int c = 0; c < d; ++c) ss += orow[c] * orow[c];
        const double rms = sqrt(ss / d + eps);
        for (int c = 0; c < d; ++c)
            y[(size_t)r * d + c] = (orow[c] / rms) * w[c] * silu(zrow[c]);
    }
}

/*
 * A linear layer without bias, weight in the Linear layout (one row per
 * output): y[t][o] = sum_i W[o][i] * x[t][i], for T rows of x [T][n_in],
 * W [n_out][n_in], y [T][n_out]. The page applies every projection of the
 * layer this way to its input ("W @ x" per token: attn_qkv, attn_gate,
 * ssm_beta, ssm_alpha before the mixer, ssm_out after it).
 */
void gdno_linear(long T, int n_in, int n_out, const double *x, const double *W, double *y)
{
    for (long t = 0; t < T; ++t) {
        const double *xr = x + (size_t)t * n_in;
        for (int o = 0; o < n_out; ++o) {
            const double *wr = W + (size_t)o * n_in;
            double acc = 0.0;
            for (int i = 0; i < n_in; ++i) acc += wr[i] * xr[i];
            y[(size_t)t * n_out + o] = acc;
        }
    }
}

/*
 * The four input projections of the layer input x [T][hidden] (the page's
 * gated DeltaNet paragraph, with the tensor names of its section "GGUF facts
 * that differ from the HF checkpoint"):
 *   qkv = attn_qkv @ x   [T][C]      the fused stream the conv runs over
 *   z   = attn_gate @ x  [T][Hv*d]   the gate of the RMSNorm
 *   b   = ssm_beta @ x   [T][Hv]     beta logits
 *   a   = ssm_alpha @ x  [T][Hv]     alpha logits
 * with w_qkv [C][hidden], w_gate [Hv*d][hidden], w_beta, w_alpha [Hv][hidden].
 */
void gdno_in_proj(long T, int hidden, int Hqk, int Hv, int d, const double *x,
                  const double *w_qkv, const double *w_gate, const double *w_beta,
                  const double *w_alpha, double *qkv, double *z, double *b, double *a)
{
    const int C = d * (2 * Hqk + Hv);
    gdno_linear(T, hidden, C, x, w_qkv, qkv);
    gdno_linear(T, hidden, Hv * d, x, w_gate, z);
    gdno_linear(T, hidden, Hv, x, w_beta, b);
    gdno_linear(T, hidden, Hv, x, w_alpha, a);
}

/* Scalar functions, exposed so tests can pin them on their own. */
double gdno_sigmoid(double x) { return sigmoid(x); }
double gdno_softplus(double x) { return softplus(x); }
double gdno_silu(double x) { return silu(x); }
