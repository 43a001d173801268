/*
 * fmoe_oracle.c -- plain CPU reference of the quantized MoE decode layer.
 *
 * TEST INFRASTRUCTURE ONLY (see fmoe_oracle.h).  Built with -O2 and
 * -ffp-contract=off so that every expression is rounded as written.
 *
 * Page keys used in the citations below:
 *   [WAS]  "Was ist Flash-MoE? 397B-Parameter-KI-Modelle auf einem Laptop
 *          laufen lassen" (a2a-mcp.org, German) and its translations.
 *   [HADA] "Flash-MoE - Ein 397-Milliarden-Parameter-Modell auf einem
 *          Notebook ausfuehren" (news.hada.io).
 */
#include "fmoe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ format */

/* Packed codes.  [WAS] section "3. Handoptimierte Metal Compute-Shader" names
 * 4-bit and 2-bit matrix-vector kernels but no bit order; the reading taken
 * here is LSB-first: element k of a row lives in byte k*bits/8 at bit
 * position (k mod (8/bits))*bits, rows stored one after another. */
int or_code(const uint8_t *row, int bits, int64_t k)
{
    int per_byte = 8 / bits;
    uint8_t byte = row[k / per_byte];
    int shift = (int)(k % per_byte) * bits;
    return (byte >> shift) & ((1 << bits) - 1);
}

static double or_bf16_to_double(uint16_t v)
{
    uint32_t bits32 = (uint32_t)v << 16;
    float f;
    memcpy(&f, &bits32, sizeof f);
    return (double)f;
}

double or_sb(const void *arr, int sbytes, int64_t idx)
{
    if (sbytes == 2) {
        uint16_t v;
        memcpy(&v, (const uint8_t *)arr + 2 * idx, 2);
        return or_bf16_to_double(v);
    }
    float f;
    memcpy(&f, (const uint8_t *)arr + 4 * idx, 4);
    return (double)f;
}

static int64_t or_round256(int64_t v) { return (v + 255) / 256 * 256; }

/* One expert is one contiguous unit holding gate, up and down with their
 * scales and biases ([HADA] "Schluesseltechnologien / SSD Expert Streaming":
 * each loaded expert is about 6.75 MB).  Section order and 256-byte alignment
 * are this repository's layout choice. */
int64_t or_slab_layout(int H, int I, or_fmt f, int64_t off[9])
{
    /* gate and up are [I x H] (input dim H), down is [H x I] (input dim I). */
    const int64_t rows[3] = {I, I, H};
    const int64_t cols[3] = {H, H, I};
    int64_t pos = 0;
    for (int m = 0; m < 3; ++m) {
        int64_t qbytes = rows[m] * cols[m] * f.bits / 8;
        int64_t sbytes = rows[m] * (cols[m] / f.group) * f.sbytes;
        off[3 * m + 0] = pos; pos = or_round256(pos + qbytes);
        off[3 * m + 1] = pos; pos = or_round256(pos + sbytes);
        off[3 * m + 2] = pos; pos = or_round256(pos + sbytes);
    }
    return pos;
}

/* ---------------------------------------------------------------- dequant */

/* Affine dequantisation, [WAS] "2. FMA-optimierte Dequantisierungs-Kernel":
 * the weight is code * scale + bias.  Group runs along the input dim. */
void or_dequant(const uint8_t *q, const void *s, const void *b, or_fmt f,
                int N, int K, double *W)
{
    const int64_t row_bytes = (int64_t)K * f.bits / 8;
    const int64_t ng = K / f.group;
    for (int n = 0; n < N; ++n) {
        const uint8_t *row = q + (int64_t)n * row_bytes;
        for (int k = 0; k < K; ++k) {
            int64_t gi = (int64_t)n * ng + k / f.group;
            double sc = or_sb(s, f.sbytes, gi);
            double bi = or_sb(b, f.sbytes, gi);
            W[(int64_t)n * K + k] = (double)or_code(row, f.bits, k) * sc + bi;
        }
    }
}

void or_gemv_dense(const double *W, int N, int K, const double *x, double *y)
{
    for (int n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int k = 0; k < K; ++k)
            acc += W[(int64_t)n * K + k] * x[k];
        y[n] = acc;
    }
}

void or_gemv(const uint8_t *q, const void *s, const void *b, or_fmt f,
             int N, int K, const double *x, double *y)
{
    double *W = (double *)malloc(sizeof(double) * (size_t)N * (size_t)K);
    if (!W) { for (int n = 0; n < N; ++n) y[n] = NAN; return; }
    or_dequant(q, s, b, f, N, K, W);
    or_gemv_dense(W, N, K, x, y);
    free(W);
}

/* [WAS] "2. FMA-optimierte Dequantisierungs-Kernel": precompute scale*x and
 * bias*x, then one fused multiply-add per code. */
void or_gemv_fma_form(const uint8_t *q, const void *s, const void *b, or_fmt f,
                      int N, int K, const double *x, double *y)
{
    const int64_t row_bytes = (int64_t)K * f.bits / 8;
    const int64_t ng = K / f.group;
    for (int n = 0; n < N; ++n) {
        const uint8_t *row = q + (int64_t)n * row_bytes;
        double acc = 0.0;
        for (int k = 0; k < K; ++k) {
            int64_t gi = (int64_t)n * ng + k / f.group;
            double sx = or_sb(s, f.sbytes, gi) * x[k];
            double bx = or_sb(b, f.sbytes, gi) * x[k];
            acc += fma((double)or_code(row, f.bits, k), sx, bx);
        }
        y[n] = acc;
    }
}

/* Same product with scale and bias pulled out of each group:
 * y_n = sum_g s_g * (sum_{k in g} q_k x_k) + b_g * (sum_{k in g} x_k). */
void or_gemv_groupsum(const uint8_t *q, const void *s, const void *b, or_fmt f,
                      int N, int K, const double *x, double *y)
{
    const int64_t row_bytes = (int64_t)K * f.bits / 8;
    const int64_t ng = K / f.group;
    for (int n = 0; n < N; ++n) {
        const uint8_t *row = q + (int64_t)n * row_bytes;
        double acc = 0.0;
        for (int64_t g = 0; g < ng; ++g) {
            double qx = 0.0, xs = 0.0;
            for (int j = 0; j < f.group; ++j) {
                int64_t k = g * f.group + j;
                qx += (double)or_code(row, f.bits, k) * x[k];
                xs += x[k];
            }
            acc += or_sb(s, f.sbytes, (int64_t)n * ng + g) * qx
                 + or_sb(b, f.sbytes, (int64_t)n * ng + g) * xs;
        }
        y[n] = acc;
    }
}

/* The unfused form that [WAS] "2. FMA-optimierte Dequantisierungs-Kernel"
 * starts from: each weight is dequantised on its own, then multiplied by its
 * input and accumulated, all in fp32 and in input order. */
void or_gemv_naive_f32(const uint8_t *q, const void *s, const void *b, or_fmt f,
                       int N, int K, const float *x, float *y)
{
    const int64_t row_bytes = (int64_t)K * f.bits / 8;
    const int64_t ng = K / f.group;
    for (int n = 0; n < N; ++n) {
        const uint8_t *row = q + (int64_t)n * row_bytes;
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) {
            int64_t gi = (int64_t)n * ng + k / f.group;
            float sc = (float)or_sb(s, f.sbytes, gi);
            float bi = (float)or_sb(b, f.sbytes, gi);
            float wv = (float)or_code(row, f.bits, k) * sc + bi;
            acc = acc + wv * x[k];
        }
        y[n] = acc;
    }
}

/* ----------------------------------------------------------------- router */

typedef struct { double v; int32_t e; } or_pair;

/* Order: larger logit first; equal logits -> lower expert index first. */
static int or_pair_cmp(const void *pa, const void *pb)
{
    const or_pair *a = (const or_pair *)pa, *b = (const or_pair *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->e > b->e) - (a->e < b->e);
}

/* [WAS] "Verstaendnis von Mixture-of-Experts (MoE) ...": per layer a router
 * picks 4 routed experts plus 1 shared one out of 512.  Read here as: linear
 * router logits, full softmax, the k largest by full sort (lower index wins a
 * tie), weights renormalised over the selection. */
int or_route(const float *Wr, const float *x, int T, int H, int E, int k,
             int32_t *idx, double *w, double *logits, double *gap)
{
    int status = 0;
    double *l = (double *)malloc(sizeof(double) * (size_t)E);
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    or_pair *pr = (or_pair *)malloc(sizeof(or_pair) * (size_t)E);
    if (!l || !p || !pr) { free(l); free(p); free(pr); return -2; }

    for (int t = 0; t < T; ++t) {
        const float *xt = x + (int64_t)t * H;
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int hh = 0; hh < H; ++hh)
                acc += (double)Wr[(int64_t)e * H + hh] * (double)xt[hh];
            l[e] = acc;
            if (logits) logits[(int64_t)t * E + e] = acc;
        }
        for (int e = 0; e < E; ++e) { pr[e].v = l[e]; pr[e].e = e; }
        qsort(pr, (size_t)E, sizeof(or_pair), or_pair_cmp);

        /* softmax over all E experts (max subtracted) */
        double mx = pr[0].v, z = 0.0;
        for (int e = 0; e < E; ++e) { p[e] = exp(l[e] - mx); z += p[e]; }
        for (int e = 0; e < E; ++e) p[e] /= z;

        double zsel = 0.0;
        for (int i = 0; i < k; ++i) zsel += p[pr[i].e];
        /* the same weights from a softmax over the k selected logits only */
        double zk = 0.0;
        for (int i = 0; i < k; ++i) zk += exp(pr[i].v - mx);
        for (int i = 0; i < k; ++i) {
            double wi = p[pr[i].e] / zsel;
            double wd = exp(pr[i].v - mx) / zk;
            if (fabs(wi - wd) > 1e-12) status = -1;
            if (idx) idx[(int64_t)t * k + i] = pr[i].e;
            if (w) w[(int64_t)t * k + i] = wi;
        }
        if (gap) gap[t] = (k < E) ? pr[k - 1].v - pr[k].v : INFINITY;
    }
    free(l); free(p); free(pr);
    return status;
}

void or_topk_kpass(const double *logits, int E, int k, int32_t *idx)
{
    unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
    if (!taken) return;
    for (int i = 0; i < k; ++i) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || logits[e] > logits[best]) best = e;  /* strict: first index wins */
        }
        idx[i] = best;
        taken[best] = 1;
    }
    free(taken);
}

/* ------------------------------------------------------------- expert FFN */

/* [WAS] "3. Handoptimierte Metal Compute-Shader" lists a fused SwiGLU
 * activation; the standard reading is silu(gate) * up with
 * silu(z) = z * sigmoid(z). */
double or_silu(double z) { return z / (1.0 + exp(-z)); }

void or_expert_ffn(const uint8_t *slab, int H, int I, or_fmt f,
                   const double *x, double *y)
{
    int64_t off[9];
    or_slab_layout(H, I, f, off);
    double *gt = (double *)malloc(sizeof(double) * (size_t)I);
    double *up = (double *)malloc(sizeof(double) * (size_t)I);
    double *a = (double *)malloc(sizeof(double) * (size_t)I);
    if (!gt || !up || !a) { free(gt); free(up); free(a); for (int m = 0; m < H; ++m) y[m] = NAN; return; }
    or_gemv(slab + off[0], slab + off[1], slab + off[2], f, I, H, x, gt);
    or_gemv(slab + off[3], slab + off[4], slab + off[5], f, I, H, x, up);
    for (int n = 0; n < I; ++n) a[n] = or_silu(gt[n]) * up[n];
    or_gemv(slab + off[6], slab + off[7], slab + off[8], f, H, I, a, y);
    free(gt); free(up); free(a);
}

/* [WAS] "3. Handoptimierte Metal Compute-Shader": two-phase RMSNorm, sum of
 * squares first, then applied. */
void or_rmsnorm(const double *h, const float *gamma, int H, double eps, double *y)
{
    double ss = 0.0;
    for (int m = 0; m < H; ++m) ss += h[m] * h[m];
    double inv = 1.0 / sqrt(ss / (double)H + eps);
    for (int m = 0; m < H; ++m) y[m] = (double)gamma[m] * h[m] * inv;
}

/* [WAS] "3. Handoptimierte Metal Compute-Shader": the MoE combine, residual
 * and sigmoid gating happen in one pass; [HADA] "Deferred GPU Expert
 * Compute": combine, normalisation and residual feed the next layer. */
void or_moe_token(const uint8_t *const *routed, const double *w, int k,
                  const uint8_t *shared, int H, int I, or_fmt f,
                  const float *wsg, const float *gamma, double eps,
                  const float *x, const float *r,
                  double *g_out, double *moe, double *h, double *y)
{
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    double *ye = (double *)malloc(sizeof(double) * (size_t)H);
    if (!xd || !ye) { free(xd); free(ye); return; }
    for (int m = 0; m < H; ++m) { xd[m] = (double)x[m]; moe[m] = 0.0; }

    for (int i = 0; i < k; ++i) {
        or_expert_ffn(routed[i], H, I, f, xd, ye);
        for (int m = 0; m < H; ++m) moe[m] += w[i] * ye[m];
    }
    double gl = 0.0;
    for (int m = 0; m < H; ++m) gl += (double)wsg[m] * xd[m];
    double g = 1.0 / (1.0 + exp(-gl));
    or_expert_ffn(shared, H, I, f, xd, ye);
    for (int m = 0; m < H; ++m) moe[m] += g * ye[m];
    for (int m = 0; m < H; ++m) h[m] = (double)r[m] + moe[m];
    or_rmsnorm(h, gamma, H, eps, y);
    if (g_out) *g_out = g;
    free(xd); free(ye);
}

int or_layer_forward(const float *Wr, const uint8_t *slabs, int64_t slab_stride,
                     const float *wsg, const float *gamma, double eps,
                     int H, int I, int E, int k, or_fmt f, int T,
                     const float *x, const float *r, const int32_t *forced_idx,
                     int32_t *idx, double *w, double *logits, double *gap,
                     double *g, double *moe, double *h, double *y)
{
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)T * (size_t)k);
    double *ww = (double *)malloc(sizeof(double) * (size_t)T * (size_t)k);
    double *lg = (double *)malloc(sizeof(double) * (size_t)T * (size_t)E);
    double *mo = (double *)malloc(sizeof(double) * (size_t)H);
    double *hh = (double *)malloc(sizeof(double) * (size_t)H);
    double *yy = (double *)malloc(sizeof(double) * (size_t)H);
    const uint8_t **rp = (const uint8_t **)malloc(sizeof(uint8_t *) * (size_t)k);
    if (!sel || !ww || !lg || !mo || !hh || !yy || !rp) {
        free(sel); free(ww); free(lg); free(mo); free(hh); free(yy); free(rp);
        return -2;
    }
    int status = or_route(Wr, x, T, H, E, k, sel, ww, lg, gap);
    if (forced_idx) {
        for (int t = 0; t < T; ++t) {
            const int32_t *fi = forced_idx + (int64_t)t * k;
            double mx = -INFINITY, z = 0.0;
            for (int i = 0; i < k; ++i) {
                double v = lg[(int64_t)t * E + fi[i]];
                if (v > mx) mx = v;
            }
            for (int i = 0; i < k; ++i) z += exp(lg[(int64_t)t * E + fi[i]] - mx);
            for (int i = 0; i < k; ++i) {
                sel[(int64_t)t * k + i] = fi[i];
                ww[(int64_t)t * k + i] = exp(lg[(int64_t)t * E + fi[i]] - mx) / z;
            }
        }
    }
    for (int t = 0; t < T; ++t) {
        for (int i = 0; i < k; ++i)
            rp[i] = slabs + (int64_t)sel[(int64_t)t * k + i] * slab_stride;
        double gt;
        or_moe_token(rp, ww + (int64_t)t * k, k, slabs + (int64_t)E * slab_stride,
                     H, I, f, wsg, gamma, eps,
                     x + (int64_t)t * H, r + (int64_t)t * H, &gt, mo, hh, yy);
        if (g) g[t] = gt;
        for (int m = 0; m < H; ++m) {
            if (moe) moe[(int64_t)t * H + m] = mo[m];
            if (h) h[(int64_t)t * H + m] = hh[m];
            if (y) y[(int64_t)t * H + m] = yy[m];
        }
    }
    if (idx) memcpy(idx, sel, sizeof(int32_t) * (size_t)T * (size_t)k);
    if (w) memcpy(w, ww, sizeof(double) * (size_t)T * (size_t)k);
    if (logits) memcpy(logits, lg, sizeof(double) * (size_t)T * (size_t)E);
    free(sel); free(ww); free(lg); free(mo); free(hh); free(yy); free(rp);
    return status;
}
