/*
 * fmoe_oracle.h -- plain, slow CPU reference of the quantized MoE decode layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (libfmoe.so and its Python binding) never links, imports or calls it, and
 * this code shares nothing with the GPU path: its own unpacking, its own slab
 * layout arithmetic, its own bf16 widening, its own sort.
 *
 * Everything is computed in fp64 from exactly widened inputs (fp32 -> fp64,
 * bf16 -> fp32 by placing the 16 stored bits in the high half).  The layer is
 * written as the plain definition -- dequantise, multiply, sort, softmax --
 * with no blocking, fusion or reordering.
 *
 * Sources (web pages on the Flash-MoE engine):
 *   [WAS]  "Was ist Flash-MoE? 397B-Parameter-KI-Modelle auf einem Laptop
 *          laufen lassen" (a2a-mcp.org blog, German), and its zh/hi/pt
 *          translations.
 *   [HADA] "Flash-MoE - Ein 397-Milliarden-Parameter-Modell auf einem
 *          Notebook ausfuehren" (news.hada.io summary).
 * Readings of points the pages leave open are listed beside the function that
 * takes them.
 *
 * Parity pins: every function here is checked by CPU tests against closed
 * forms, brute force or the pages' printed size figures; none is marked
 * "parity unpinned".
 */
#ifndef FMOE_ORACLE_H
#define FMOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Quantisation format: bits in {2,4}; group size along the input dim;
 * sbytes = 4 (fp32 scale/bias) or 2 (bf16 scale/bias). */
typedef struct {
    int32_t bits;
    int32_t group;
    int32_t sbytes;
} or_fmt;

/* Unsigned code of element k of a packed row (LSB-first within each byte). */
int or_code(const uint8_t *row, int bits, int64_t k);

/* Widen one stored scale or bias (index idx of its array) to fp64. */
double or_sb(const void *arr, int sbytes, int64_t idx);

/* Canonical expert slab: gate.q gate.s gate.b up.q up.s up.b down.q down.s
 * down.b, each section starting on a 256-byte boundary.  off[9] receives the
 * section offsets, the return value is the slab size (a multiple of 256). */
int64_t or_slab_layout(int H, int I, or_fmt f, int64_t off[9]);

/* deq(W)[n,k] = q[n,k] * s[n,k/G] + b[n,k/G]  into the dense N x K array W. */
void or_dequant(const uint8_t *q, const void *s, const void *b, or_fmt f,
                int N, int K, double *W);

/* Textbook dense GEMV on an fp64 matrix. */
void or_gemv_dense(const double *W, int N, int K, const double *x, double *y);

/* The quantised GEMV by its definition: dequantise, then multiply. */
void or_gemv(const uint8_t *q, const void *s, const void *b, or_fmt f,
             int N, int K, const double *x, double *y);

/* The pages' rearranged form: sum_k fma(q, s*x_k, b*x_k), fp64. */
void or_gemv_fma_form(const uint8_t *q, const void *s, const void *b, or_fmt f,
                      int N, int K, const double *x, double *y);

/* Group-sum form: sum_g s_g * sum_{k in g} q x_k + b_g * sum_{k in g} x_k. */
void or_gemv_groupsum(const uint8_t *q, const void *s, const void *b, or_fmt f,
                      int N, int K, const double *x, double *y);

/* The pages' "before" form in fp32: acc += (q*s + b) * x, sequential. */
void or_gemv_naive_f32(const uint8_t *q, const void *s, const void *b, or_fmt f,
                       int N, int K, const float *x, float *y);

/* Router for T tokens.  logits[t,e] = sum_h Wr[e,h] x[t,h] (fp64); the k
 * selected experts ordered by (logit desc, index asc) from a full sort;
 * weights = softmax over all E, renormalised over the selection; gap =
 * logit of the k-th minus the (k+1)-th (or +inf when k == E).
 * Returns 0, or -1 if the renormalised weights and a direct softmax over
 * the selected logits disagree by more than 1e-12. */
int or_route(const float *Wr, const float *x, int T, int H, int E, int k,
             int32_t *idx, double *w, double *logits, double *gap);

/* Top-k by k passes of arg-max (first index wins ties), for cross-checks. */
void or_topk_kpass(const double *logits, int E, int k, int32_t *idx);

/* silu(z) = z / (1 + exp(-z)). */
double or_silu(double z);

/* One expert FFN: a = silu(deq(Wg) x) * (deq(Wu) x); y = deq(Wd) a. */
void or_expert_ffn(const uint8_t *slab, int H, int I, or_fmt f,
                   const double *x, double *y);

/* y = gamma * h / sqrt(mean(h^2) + eps). */
void or_rmsnorm(const double *h, const float *gamma, int H, double eps, double *y);

/* One token of the MoE layer given its routing:
 *   moe = sum_i w_i * FFN_{idx_i}(x) + g * FFN_shared(x),  g = sigmoid(wsg . x)
 *   h   = r + moe,   y = RMSNorm(h).
 * routed[i] points at the slab of expert idx_i, shared at the shared slab. */
void or_moe_token(const uint8_t *const *routed, const double *w, int k,
                  const uint8_t *shared, int H, int I, or_fmt f,
                  const float *wsg, const float *gamma, double eps,
                  const float *x, const float *r,
                  double *g_out, double *moe, double *h, double *y);

/* Whole layer for T tokens (route, then or_moe_token per token).  slabs holds
 * E+1 expert slabs of slab_stride bytes each; slab E is the shared expert.
 * If forced_idx is non-NULL it replaces the router's selection (weights are
 * then the softmax over the forced experts' logits).  Any of the optional
 * outputs may be NULL.  Returns or_route's status. */
int or_layer_forward(const float *Wr, const uint8_t *slabs, int64_t slab_stride,
                     const float *wsg, const float *gamma, double eps,
                     int H, int I, int E, int k, or_fmt f, int T,
                     const float *x, const float *r, const int32_t *forced_idx,
                     int32_t *idx, double *w, double *logits, double *gap,
                     double *g, double *moe, double *h, double *y);

#ifdef __cplusplus
}
#endif

#endif
