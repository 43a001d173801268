/*
 * fmoe_oracle_next.c -- plain CPU references of the Gated DeltaNet state update
 * and of full-attention decode with rotary embedding (fmoe_oracle_next.h).
 *
 * TEST INFRASTRUCTURE ONLY.  Built with -O2 and -ffp-contract=off, in fp64.
 *
 * Page key: [WAS] "Was ist Flash-MoE? 397B-Parameter-KI-Modelle auf einem
 * Laptop laufen lassen" (a2a-mcp.org, German) and its translations.
 */
#include "fmoe_oracle_next.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* -------------------------------------------------------- Gated DeltaNet */

/* The four steps in the order the section names its BLAS calls: scale the
 * state (sscal), read the value the state holds for the key (sgemv), write the
 * difference to the new value along the key (sger), read the output for the
 * query (sgemv). */
void or_deltanet_step(const float *q, const float *k, const float *v, const float *a,
                      const float *beta, const float *state_in, int B, int NH, int dk, int dv,
                      double *state_out, double *out)
{
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < NH; ++h) {
            const size_t bh = (size_t)b * NH + h;
            const float *qh = q + bh * dk, *kh = k + bh * dk, *vh = v + bh * dv;
            const float *S0 = state_in + bh * dk * dv;
            double *S = state_out + bh * dk * dv;
            /* S <- a S */
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    S[(size_t)i * dv + j] = (double)a[bh] * (double)S0[(size_t)i * dv + j];
            /* u = S^T k */
            for (int j = 0; j < dv; ++j) {
                double s = 0.0;
                for (int i = 0; i < dk; ++i) s += S[(size_t)i * dv + j] * (double)kh[i];
                u[j] = s;
            }
            /* S <- S + beta k (v - u)^T */
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    S[(size_t)i * dv + j] += (double)beta[bh] * (double)kh[i] * ((double)vh[j] - u[j]);
            /* o = S^T q */
            for (int j = 0; j < dv; ++j) {
                double s = 0.0;
                for (int i = 0; i < dk; ++i) s += S[(size_t)i * dv + j] * (double)qh[i];
                out[bh * dv + j] = s;
            }
        }
    }
    free(u);
}

/* ------------------------------------------------------------- attention */

static double or_bf16(uint16_t v)
{
    uint32_t bits32 = (uint32_t)v << 16;
    float f;
    memcpy(&f, &bits32, sizeof f);
    return (double)f;
}

void or_rope_deinterleave(const float *x, int D, int pos, double base, double *y)
{
    const int half = D / 2;
    for (int i = 0; i < half; ++i) {
        const double theta = (double)pos * pow(base, -2.0 * (double)i / (double)D);
        const double c = cos(theta), s = sin(theta);
        const double x0 = (double)x[2 * i], x1 = (double)x[2 * i + 1];
        y[i] = x0 * c - x1 * s;
        y[i + half] = x0 * s + x1 * c;
    }
}

void or_attention_decode(const float *q, const uint16_t *kc, const uint16_t *vc,
                         const int32_t *len, int B, int NQ, int NKV, int D, int cap,
                         double base, double *out)
{
    const int group = NQ / NKV;
    double *qr = (double *)malloc(sizeof(double) * (size_t)D);
    double *sc = (double *)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
    for (int b = 0; b < B; ++b) {
        const int L = len[b];
        for (int h = 0; h < NQ; ++h) {
            const int hk = h / group;
            const size_t base_kv = ((size_t)b * NKV + hk) * (size_t)cap * D;
            double *o = out + ((size_t)b * NQ + h) * D;
            or_rope_deinterleave(q + ((size_t)b * NQ + h) * D, D, L - 1, base, qr);
            /* scores */
            double mx = -INFINITY;
            for (int t = 0; t < L; ++t) {
                double s = 0.0;
                for (int d = 0; d < D; ++d) s += qr[d] * or_bf16(kc[base_kv + (size_t)t * D + d]);
                sc[t] = s / sqrt((double)D);
                if (sc[t] > mx) mx = sc[t];
            }
            /* softmax */
            double z = 0.0;
            for (int t = 0; t < L; ++t) {
                sc[t] = exp(sc[t] - mx);
                z += sc[t];
            }
            /* weighted values */
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            for (int t = 0; t < L; ++t) {
                const double p = sc[t] / z;
                for (int d = 0; d < D; ++d) o[d] += p * or_bf16(vc[base_kv + (size_t)t * D + d]);
            }
        }
    }
    free(qr);
    free(sc);
}
