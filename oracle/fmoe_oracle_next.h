/*
 * fmoe_oracle_next.h -- plain CPU references of the two non-MoE decode steps
 * the pages describe beside the MoE layer: the Gated DeltaNet state update and
 * full-attention decode with rotary position embedding.
 *
 * TEST INFRASTRUCTURE ONLY, like fmoe_oracle.h: the tests, the smoke check and
 * the CPU-baseline leg of the benchmark call it; the library never does.
 * Everything is computed in fp64 from the stored inputs.
 */
#ifndef FMOE_ORACLE_NEXT_H
#define FMOE_ORACLE_NEXT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One decode step of the Gated DeltaNet recurrence for B sequences x NH heads
 * ([WAS] "4. Accelerate BLAS fuer Gated DeltaNet-Schichten": the state matrix
 * of each of the 64 heads is updated with a scale, a matrix-vector product and
 * a rank-1 update).  Per (b, h), with the head's state S [dk x dv] (row i,
 * column j), key k and query q [dk], value v [dv], decay a and write strength
 * beta:
 *   S <- a S;   u = S^T k;   S <- S + beta k (v - u)^T;   o = S^T q.
 * state_in / state_out: [B, NH, dk, dv] (state_out in fp64), q, k: [B, NH, dk],
 * v: [B, NH, dv], a, beta: [B, NH], out: [B, NH, dv] (fp64). */
void or_deltanet_step(const float *q, const float *k, const float *v, const float *a,
                      const float *beta, const float *state_in, int B, int NH, int dk, int dv,
                      double *state_out, double *out);

/* Rotary position embedding of one head vector x [D] at position pos, with the
 * input's rotation pairs interleaved (x[2i], x[2i+1]) and the output in
 * half-split order (pair i lands at i and i + D/2):
 *   theta_i = pos * base^(-2i/D)
 *   y[i]       = x[2i] cos theta_i - x[2i+1] sin theta_i
 *   y[i + D/2] = x[2i] sin theta_i + x[2i+1] cos theta_i
 * ([WAS] "3. Handoptimierte Metal Compute-Shader": RoPE on the GPU with the
 * query de-interleaved). */
void or_rope_deinterleave(const float *x, int D, int pos, double base, double *y);

/* Decode attention of one new token for B sequences ([WAS] section 3: batched
 * attention for the full-attention layers; [WAS] "Wichtige Erkenntnisse" and
 * the layer list: Q K^T, softmax, scores V).  Per sequence b: its query
 * heads q [NQ, D] (interleaved pairs, rotated here with or_rope_deinterleave at
 * position len[b] - 1), a cache of len[b] keys and values per KV head, stored
 * as bf16 bits [B, NKV, cap, D] (keys already rotated, half-split order).  Query
 * head h reads KV head h / (NQ / NKV):
 *   s_t = (q_rot . K_t) / sqrt(D),   p = softmax(s),   o_h = sum_t p_t V_t.
 * out: [B, NQ, D] (fp64). */
void or_attention_decode(const float *q, const uint16_t *kc, const uint16_t *vc,
                         const int32_t *len, int B, int NQ, int NKV, int D, int cap,
                         double base, double *out);

#ifdef __cplusplus
}
#endif

#endif
