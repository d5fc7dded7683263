/* oracle.c -- plain CPU reference for the quantized MoE feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library or its binding.
 *
 * The layer (router -> top-k experts with softmax gates -> gated FFN per
 * selected expert -> weighted combine, plus an optional dense shared expert)
 * is the MoE block the pages describe: the Camelid README ("Gemma 4" section:
 * 128 experts, top-8 sparse branch plus a dense shared expert; "Experimental
 * lanes": exact expert-probability ties go to the lower index) and the
 * TurboFieldfare summary ("memory and expert streaming": router-chosen
 * experts, a shared branch computed alongside, prefill in chunks of at most
 * 128 tokens).  The pages give no formulas; each function below writes out
 * the plain definition it uses.
 *
 * Precision: every weight is decoded to its exact value, every contraction is
 * summed sequentially in double, and a result is rounded to fp32 once.  The
 * optional OpenMP loops run over independent outputs only, so the result is
 * bitwise the same for any thread count.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;

int or_set_threads(int n) {
    if (n < 1) n = 1;
#ifdef _OPENMP
    g_threads = n;
#else
    g_threads = 1;
#endif
    return g_threads;
}

int or_get_threads(void) { return g_threads; }

/* ---------------------------------------------------------------- formats */

int or_row_bytes(int fmt, int cols) {
    switch (fmt) {
    case OR_Q8_0: return cols % 32 ? -1 : cols / 32 * 34;
    case OR_Q4_0: return cols % 32 ? -1 : cols / 32 * 18;
    case OR_I8_ROW: return cols;
    case OR_I4_ROW: return cols % 2 ? -1 : cols / 2;
    case OR_Q4_1: return cols % 32 ? -1 : cols / 32 * 20;
    case OR_I2_ROW: return cols % 4 ? -1 : cols / 4;
    default: return -1;
    }
}

/* IEEE 754 binary16 -> double, written out from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 holds
 * the subnormals fraction * 2^-24. */
static double half_value(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an fp32 bit pattern. */
static double bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Decode one row to exact weight values.
 *   Q8_0:  blocks of 34 bytes = fp16 d, 32 x int8 q;          w = d * q
 *   Q4_0:  blocks of 18 bytes = fp16 d, 16 bytes of nibbles;  weight j is the
 *          low nibble of byte j, weight j+16 its high nibble;  w = d * (n - 8)
 *   I8_ROW: int8 q per weight, fp32 scale s per row;          w = s * q
 *   I4_ROW: byte j holds weight 2j (low nibble) and 2j+1 (high nibble) as
 *          two's-complement 4-bit integers v in [-8, 7];      w = s * v
 *   Q4_1:  blocks of 20 bytes = fp16 d, fp16 m, 16 bytes of nibbles in the
 *          Q4_0 order, codes n in 0..15 without offset;       w = d * n + m
 *   I2_ROW: byte j holds weights 4j..4j+3, weight 4j+i in bits 2i..2i+1, as
 *          two's-complement 2-bit integers v in [-2, 1];      w = s * v
 * All products are exact in double, and so is the Q4_1 sum: d * n and m are
 * both multiples of 2^-24 (the smallest binary16 step) below 2^21, so their
 * sum needs at most 45 significant bits. */
int or_decode_row(int fmt, const uint8_t *row, float scale, int K, double *w) {
    if (!row || !w || K <= 0 || or_row_bytes(fmt, K) < 0) return OR_EINVAL;
    if (fmt == OR_Q8_0) {
        for (int b = 0; b < K / 32; ++b) {
            const uint8_t *blk = row + 34 * b;
            double d = half_value((uint16_t)(blk[0] | (blk[1] << 8)));
            for (int i = 0; i < 32; ++i) w[32 * b + i] = d * (double)(int8_t)blk[2 + i];
        }
    } else if (fmt == OR_Q4_0) {
        for (int b = 0; b < K / 32; ++b) {
            const uint8_t *blk = row + 18 * b;
            double d = half_value((uint16_t)(blk[0] | (blk[1] << 8)));
            for (int j = 0; j < 16; ++j) {
                int lo = blk[2 + j] & 15, hi = blk[2 + j] >> 4;
                w[32 * b + j] = d * (double)(lo - 8);
                w[32 * b + j + 16] = d * (double)(hi - 8);
            }
        }
    } else if (fmt == OR_Q4_1) {
        for (int b = 0; b < K / 32; ++b) {
            const uint8_t *blk = row + 20 * b;
            double d = half_value((uint16_t)(blk[0] | (blk[1] << 8)));
            double m = half_value((uint16_t)(blk[2] | (blk[3] << 8)));
            for (int j = 0; j < 16; ++j) {
                w[32 * b + j] = d * (double)(blk[4 + j] & 15) + m;
                w[32 * b + j + 16] = d * (double)(blk[4 + j] >> 4) + m;
            }
        }
    } else if (fmt == OR_I2_ROW) {
        for (int j = 0; j < K / 4; ++j) {
            for (int i = 0; i < 4; ++i) {
                int c = (row[j] >> (2 * i)) & 3;
                w[4 * j + i] = (double)scale * (double)(c >= 2 ? c - 4 : c);
            }
        }
    } else if (fmt == OR_I8_ROW) {
        for (int c = 0; c < K; ++c) w[c] = (double)scale * (double)(int8_t)row[c];
    } else { /* OR_I4_ROW */
        for (int j = 0; j < K / 2; ++j) {
            int lo = row[j] & 15, hi = row[j] >> 4;
            int vlo = lo >= 8 ? lo - 16 : lo, vhi = hi >= 8 ? hi - 16 : hi;
            w[2 * j] = (double)scale * (double)vlo;
            w[2 * j + 1] = (double)scale * (double)vhi;
        }
    }
    return OR_OK;
}

static int qmat_ok(const or_qmat *W) {
    if (!W || !W->data || W->rows <= 0 || W->cols <= 0) return 0;
    if (or_row_bytes(W->fmt, W->cols) < 0) return 0;
    if ((W->fmt == OR_I8_ROW || W->fmt == OR_I4_ROW || W->fmt == OR_I2_ROW) && !W->scales) return 0;
    return 1;
}

static float row_scale(const or_qmat *W, int r) {
    return (W->fmt == OR_I8_ROW || W->fmt == OR_I4_ROW || W->fmt == OR_I2_ROW) ? W->scales[r] : 0.0f;
}

static const uint8_t *row_ptr(const or_qmat *W, int r) {
    return W->data + (size_t)r * (size_t)or_row_bytes(W->fmt, W->cols);
}

/* ---------------------------------------------------------------- GEMV */

/* y[b][r] = fl32( sum_{c=0}^{K-1} w[r][c] * x[b][c] ), summed in order c = 0..K-1
 * in double; S[b][r] = sum_c |w[r][c] * x[b][c]| (the tolerance basis). */
int or_qgemv(const or_qmat *W, int xtype, const void *x, int B, float *y, double *S) {
    if (!qmat_ok(W) || !x || !y || B <= 0) return OR_EINVAL;
    if (xtype != OR_X_F32 && xtype != OR_X_BF16) return OR_EINVAL;
    const int N = W->rows, K = W->cols;
    double *xd = (double *)malloc(sizeof(double) * (size_t)B * K);
    if (!xd) return OR_EINVAL;
    for (size_t i = 0; i < (size_t)B * K; ++i)
        xd[i] = xtype == OR_X_F32 ? (double)((const float *)x)[i] : bf16_value(((const uint16_t *)x)[i]);
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int r = 0; r < N; ++r) {
        double *w = (double *)malloc(sizeof(double) * (size_t)K);
        if (!w) { bad = 1; continue; }
        or_decode_row(W->fmt, row_ptr(W, r), row_scale(W, r), K, w);
        for (int b = 0; b < B; ++b) {
            const double *xb = xd + (size_t)b * K;
            double acc = 0.0, s = 0.0;
            for (int c = 0; c < K; ++c) {
                double p = w[c] * xb[c];
                acc += p;
                s += fabs(p);
            }
            y[(size_t)b * N + r] = (float)acc;
            if (S) S[(size_t)b * N + r] = s;
        }
        free(w);
    }
    free(xd);
    return bad ? OR_EINVAL : OR_OK;
}

/* ---------------------------------------------------------------- router */

/* Top-k by repeated selection: slot j takes the largest logit not yet taken;
 * among equal logits the lower expert index wins (the exact-tie rule of the
 * Camelid README, "Experimental lanes").  IEEE comparison, so -0 == +0. */
static void select_topk(const float *l, int E, int k, int32_t *idx, unsigned char *taken) {
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || l[e] > l[best] || (l[e] == l[best] && e < best)) best = e;
        }
        taken[best] = 1;
        idx[j] = best;
    }
}

/* logit[t][e] = fl32( sum_c Wr[e][c] x[t][c] + bias[e] )  (double sum)
 * gates: softmax over the k selected logits, g_j = exp(l_j - l_0) / sum_i exp(l_i - l_0),
 * evaluated in double and rounded to fp32. */
int or_route_topk(const float *x, int T, int H, const float *Wr, const float *bias,
                  int E, int k, int32_t *idx, float *gates, float *logits, float *margin) {
    if (!x || !Wr || !idx || !gates || T <= 0 || H <= 0 || E <= 0 || k <= 0 || k > E)
        return OR_EINVAL;
    float *l = (float *)malloc(sizeof(float) * (size_t)T * E);
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    if (!l || !taken) { free(l); free(taken); return OR_EINVAL; }
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int te = 0; te < T * E; ++te) {
        int t = te / E, e = te % E;
        double acc = 0.0;
        for (int c = 0; c < H; ++c) acc += (double)Wr[(size_t)e * H + c] * (double)x[(size_t)t * H + c];
        if (bias) acc += (double)bias[e];
        l[te] = (float)acc;
    }
    int rc = OR_OK;
    for (int i = 0; i < T * E; ++i)
        if (!isfinite(l[i])) rc = OR_ENONFINITE;
    if (rc == OR_OK) {
        for (int t = 0; t < T; ++t) {
            const float *lt = l + (size_t)t * E;
            int32_t *it = idx + (size_t)t * k;
            select_topk(lt, E, k, it, taken);
            double m = lt[it[0]], z = 0.0;
            for (int j = 0; j < k; ++j) z += exp((double)lt[it[j]] - m);
            for (int j = 0; j < k; ++j) gates[(size_t)t * k + j] = (float)(exp((double)lt[it[j]] - m) / z);
            if (margin) {
                float best_out = -INFINITY;
                int any = 0;
                for (int e = 0; e < E; ++e)
                    if (!taken[e] && (!any || lt[e] > best_out)) { best_out = lt[e]; any = 1; }
                margin[t] = any ? lt[it[k - 1]] - best_out : INFINITY;
            }
        }
        if (logits) memcpy(logits, l, sizeof(float) * (size_t)T * E);
    }
    free(l);
    free(taken);
    return rc;
}

/* ---------------------------------------------------------------- FFN */

/* GELU, tanh form (Hendrycks & Gimpel, "Gaussian Error Linear Units"):
 *   gelu(z) = z/2 * (1 + tanh( sqrt(2/pi) * (z + 0.044715 z^3) ))
 * SiLU (the swish gate of the GLU variants of Shazeer, "GLU Variants Improve
 * Transformer"):  silu(z) = z / (1 + exp(-z)). */
static double act_value(int act, double z) {
    if (act == OR_ACT_SILU) return z / (1.0 + exp(-z));
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
}

/* One token through a gated FFN, all in double:
 *   a = Wg x,  u = Wu x,  h = act(a) * u,  o = Wd h,  s = sum |Wd[i][f] h[f]|. */
static int ffn_token(const or_qmat *g, const or_qmat *u, const or_qmat *d, int act,
                     const double *x, double *h, double *o, double *s) {
    const int F = g->rows, H = g->cols;
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int f = 0; f < F; ++f) {
        double *w = (double *)malloc(sizeof(double) * (size_t)H);
        if (!w) { bad = 1; continue; }
        double a = 0.0, b = 0.0;
        or_decode_row(g->fmt, row_ptr(g, f), row_scale(g, f), H, w);
        for (int c = 0; c < H; ++c) a += w[c] * x[c];
        or_decode_row(u->fmt, row_ptr(u, f), row_scale(u, f), H, w);
        for (int c = 0; c < H; ++c) b += w[c] * x[c];
        h[f] = act_value(act, a) * b;
        free(w);
    }
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int i = 0; i < d->rows; ++i) {
        double *w = (double *)malloc(sizeof(double) * (size_t)F);
        if (!w) { bad = 1; continue; }
        or_decode_row(d->fmt, row_ptr(d, i), row_scale(d, i), F, w);
        double acc = 0.0, sa = 0.0;
        for (int f = 0; f < F; ++f) {
            double p = w[f] * h[f];
            acc += p;
            sa += fabs(p);
        }
        o[i] = acc;
        s[i] = sa;
        free(w);
    }
    return bad ? OR_EINVAL : OR_OK;
}

static int ffn_shapes_ok(const or_qmat *g, const or_qmat *u, const or_qmat *d) {
    if (!qmat_ok(g) || !qmat_ok(u) || !qmat_ok(d)) return 0;
    return g->rows == u->rows && g->cols == u->cols && d->cols == g->rows && d->rows == g->cols;
}

int or_ffn(const or_qmat *gate, const or_qmat *up, const or_qmat *down, int act,
           const float *x, int T, float *y, double *S) {
    if (!ffn_shapes_ok(gate, up, down) || !x || !y || T <= 0) return OR_EINVAL;
    if (act != OR_ACT_GELU_TANH && act != OR_ACT_SILU) return OR_EINVAL;
    const int H = gate->cols, F = gate->rows;
    double *xd = malloc(sizeof(double) * H), *h = malloc(sizeof(double) * F);
    double *o = malloc(sizeof(double) * H), *s = malloc(sizeof(double) * H);
    int rc = (xd && h && o && s) ? OR_OK : OR_EINVAL;
    for (int t = 0; t < T && rc == OR_OK; ++t) {
        for (int c = 0; c < H; ++c) xd[c] = x[(size_t)t * H + c];
        rc = ffn_token(gate, up, down, act, xd, h, o, s);
        for (int i = 0; i < H; ++i) {
            y[(size_t)t * H + i] = (float)o[i];
            if (S) S[(size_t)t * H + i] = s[i];
        }
    }
    free(xd); free(h); free(o); free(s);
    return rc;
}

/* ---------------------------------------------------------------- layer */

/* y[t] = fl32( sum_{j<k} g_j * o_j + o_shared )  with o_j the selected expert
 * j's FFN output (double), summed in slot order; g_j are the fp32 gates.
 * S[t][i] = sum_j g_j * s_j[i] + s_shared[i]. */
int or_moe_forward(const or_moe *L, const float *x, int T, float *y,
                   int32_t *idx, float *gates, double *S) {
    if (!L || !x || !y || !idx || !gates || T <= 0) return OR_EINVAL;
    const int H = L->H, F = L->F, E = L->E, k = L->k;
    if (H <= 0 || F <= 0 || E <= 0 || k <= 0 || k > E || !L->gate || !L->up || !L->down) return OR_EINVAL;
    if (L->act != OR_ACT_GELU_TANH && L->act != OR_ACT_SILU) return OR_EINVAL;
    int rc = or_route_topk(x, T, H, L->Wr, L->bias, E, k, idx, gates, NULL, NULL);
    if (rc != OR_OK) return rc;
    int Fh = F;
    if (L->has_shared) {
        if (!ffn_shapes_ok(&L->sh_gate, &L->sh_up, &L->sh_down) || L->sh_gate.cols != H) return OR_EINVAL;
        if (L->sh_gate.rows > Fh) Fh = L->sh_gate.rows;
    }
    double *xd = malloc(sizeof(double) * H), *h = malloc(sizeof(double) * Fh);
    double *o = malloc(sizeof(double) * H), *s = malloc(sizeof(double) * H);
    double *acc = malloc(sizeof(double) * H), *sacc = malloc(sizeof(double) * H);
    rc = (xd && h && o && s && acc && sacc) ? OR_OK : OR_EINVAL;
    for (int t = 0; t < T && rc == OR_OK; ++t) {
        for (int c = 0; c < H; ++c) { xd[c] = x[(size_t)t * H + c]; acc[c] = 0.0; sacc[c] = 0.0; }
        for (int j = 0; j < k && rc == OR_OK; ++j) {
            int e = idx[(size_t)t * k + j];
            const or_qmat *g = &L->gate[e], *u = &L->up[e], *d = &L->down[e];
            if (!g->data || !u->data || !d->data) { rc = OR_EMISSING; break; }
            if (!ffn_shapes_ok(g, u, d) || g->rows != F || g->cols != H) { rc = OR_EINVAL; break; }
            rc = ffn_token(g, u, d, L->act, xd, h, o, s);
            double gj = (double)gates[(size_t)t * k + j];
            for (int i = 0; i < H; ++i) { acc[i] += gj * o[i]; sacc[i] += gj * s[i]; }
        }
        if (rc == OR_OK && L->has_shared) {
            rc = ffn_token(&L->sh_gate, &L->sh_up, &L->sh_down, L->act, xd, h, o, s);
            for (int i = 0; i < H; ++i) { acc[i] += o[i]; sacc[i] += s[i]; }
        }
        for (int i = 0; i < H; ++i) {
            y[(size_t)t * H + i] = (float)acc[i];
            if (S) S[(size_t)t * H + i] = sacc[i];
        }
    }
    free(xd); free(h); free(o); free(s); free(acc); free(sacc);
    return rc;
}
