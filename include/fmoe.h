/*
 * fmoe.h -- C ABI of libfmoe.so: one decode step of a Mixture-of-Experts FFN
 * layer with 4-bit or 2-bit affine-quantised expert weights, on one AMD
 * Instinct MI355X (gfx950).
 *
 * The operation is the one described on the Flash-MoE pages:
 *   [WAS]  "Was ist Flash-MoE? 397B-Parameter-KI-Modelle auf einem Laptop
 *          laufen lassen" (a2a-mcp.org, German; zh/hi/pt translations)
 *   [HADA] "Flash-MoE - Ein 397-Milliarden-Parameter-Modell auf einem
 *          Notebook ausfuehren" (news.hada.io)
 * Per token: a router picks k routed experts plus one shared expert
 * ([WAS] "Verstaendnis von Mixture-of-Experts"); each expert is a
 * dequantised matrix-vector gate/up, SwiGLU, down chain over affine weights
 * w = code * scale + bias ([WAS] "2. FMA-optimierte Dequantisierungs-Kernel",
 * "3. Handoptimierte Metal Compute-Shader"); the results are combined with the
 * routing weights and a sigmoid-gated shared expert, added to the residual and
 * RMS-normalised for the next layer ([WAS] section 3, "MoE-Kombination +
 * Residual + Sigmoid-Gating"; [HADA] "Deferred GPU Expert Compute").
 *
 * Conventions common to every call
 * --------------------------------
 * Pointers: every tensor pointer is a DEVICE pointer owned by the caller.
 *   Descriptor structs (fmoe_qmat, fmoe_expert, fmoe_layer, fmoe_qformat) are
 *   host memory, read only during the call.  The library allocates and frees
 *   nothing on these paths and keeps no pointer after returning.
 * Streams: `stream` is a hipStream_t (NULL = the default stream).  Each call
 *   only enqueues kernels on it; no call copies between host and device or
 *   synchronises, so every call may be captured into a HIP graph.  Outputs are
 *   valid once the caller has synchronised with the stream.
 * Workspace: calls that take `ws` need ws_bytes >= the matching *_workspace_size
 *   value.  The workspace must be zero-filled before its first use (for example
 *   allocated with torch.zeros); every call leaves the counters it uses at zero
 *   again, so a workspace can be reused for any later call of any shape that
 *   fits.  Two calls in flight at once must use different workspaces.
 * Errors: arguments are validated on the host before anything is enqueued.  An
 *   invalid argument returns its status, enqueues nothing and sets the
 *   thread-local message returned by fmoe_last_error().  A failed launch returns
 *   FMOE_ERR_HIP with HIP's error text.  Faults during kernel execution surface
 *   at the caller's next synchronisation.  The library never aborts and no C++
 *   exception crosses this interface.  NaN and Inf inputs are propagated, not
 *   checked.
 * Quantised matrices: W[n, k] is stored row-major by output row n with the
 *   input dim k contiguous.  Codes are unsigned (0..2^bits-1) and packed
 *   LSB-first: element k of a row sits in byte k*bits/8 at bit position
 *   (k mod (8/bits))*bits.  scale and bias are [n, k/group] arrays of fp32 or
 *   bf16 (the same dtype for both); dequantised w = code * scale + bias.
 *   Supported: bits in {2, 4}; group in {32, 64}; k a multiple of group with
 *   k*bits/8 a multiple of 16; with S = k*bits/128 (16-byte segments per row),
 *   either S divides 64 or S is 64, 128 or 256.  q, scale and bias must be
 *   16-byte aligned.
 * Arithmetic: dot products accumulate in fp32.  Activations enter the
 *   dequantised products as fp16 values with a power-of-two scale per block
 *   of 32 (no overflow for any finite input); router logits accumulate in
 *   fp64 so that expert selection is exact.
 */
#ifndef FMOE_H
#define FMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FMOE_ABI_VERSION 1

typedef enum {
    FMOE_OK = 0,
    FMOE_ERR_NULL = 1,        /* a required pointer is NULL */
    FMOE_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
    FMOE_ERR_ALIGN = 3,       /* a pointer or stride is not aligned as required */
    FMOE_ERR_UNSUPPORTED = 4, /* a format or shape this build does not implement */
    FMOE_ERR_WORKSPACE = 5,   /* ws is NULL or smaller than required */
    FMOE_ERR_HIP = 6          /* a HIP launch failed */
} fmoe_status;

typedef enum { FMOE_F32 = 0, FMOE_BF16 = 1 } fmoe_dtype;

/* Quantisation format: bits in {2,4}; group in {32,64} along the input dim;
 * sdtype (fmoe_dtype) is the storage type of both scale and bias. */
typedef struct {
    int32_t bits;
    int32_t group;
    int32_t sdtype;
} fmoe_qformat;

/* One quantised matrix W[n, k] (see "Quantised matrices" above). */
typedef struct {
    const void *q;
    const void *scale;
    const void *bias;
    int32_t n;
    int32_t k;
} fmoe_qmat;

/* One expert: gate and up are [inter x hidden], down is [hidden x inter]. */
typedef struct {
    fmoe_qmat gate, up, down;
} fmoe_expert;

/* One MoE layer whose experts are stored as slabs.  An expert slab holds
 * gate.q gate.scale gate.bias up.q up.scale up.bias down.q down.scale down.bias
 * in this order, each section starting on a 256-byte boundary (offsets from
 * fmoe_slab_layout); [HADA] "SSD Expert Streaming" describes one expert as the
 * unit that is read (about 6.75 MB at hidden 4096 / inter 1024, 4-bit, which
 * this layout reproduces).  `slabs` holds n_experts + 1 slabs of slab_stride
 * bytes; slab n_experts is the shared expert. */
typedef struct {
    int32_t hidden;              /* H */
    int32_t inter;               /* I, expert intermediate size */
    int32_t n_experts;           /* E routed experts */
    int32_t top_k;               /* k routed experts per token, 1 <= k <= min(E, 16) */
    fmoe_qformat fmt;            /* format of every expert matrix */
    const float *router_w;       /* [E, H] fp32 router weights, row-major */
    const void *slabs;           /* (E+1) * slab_stride bytes, 256-byte aligned */
    int64_t slab_stride;         /* bytes, a multiple of 256, >= fmoe_slab_layout() */
    const float *shared_gate_w;  /* [H] fp32: shared-expert gate g = sigmoid(w . x) */
    const float *norm_w;         /* [H] fp32 RMSNorm weight gamma */
    float norm_eps;              /* RMSNorm epsilon (1e-6 in the configs here) */
} fmoe_layer;

/* Version of this interface (FMOE_ABI_VERSION). */
int32_t fmoe_abi_version(void);

/* Message for the last non-OK status returned on the calling thread. */
const char *fmoe_last_error(void);

/* Diagnostics: byte offset, within any workspace, of the 32-bit word that the
 * one-launch kernels set to 1 when one of their bounded waits for another
 * workgroup gives up instead of hanging (the call's outputs are then not
 * valid).  It stays 0 otherwise; the caller may read it and clear it. */
size_t fmoe_wait_timeout_offset(void);

/* Section offsets off[9] of an expert slab in the canonical layout and the
 * slab size in bytes (the return value; -1 with the message set if the
 * arguments are unsupported).  Host-only; enqueues nothing. */
int64_t fmoe_slab_layout(int32_t hidden, int32_t inter, const fmoe_qformat *fmt,
                         int64_t off[9]);

/* Router and top-k for T tokens ([WAS] "Verstaendnis von Mixture-of-Experts":
 * k routed experts chosen per token).  logits[t,e] = sum_h router_w[e,h] *
 * x[t,h], accumulated in fp64.  The k experts with the largest logits are
 * returned in idx[t, 0..k-1] ordered by (logit descending, index ascending),
 * so a tie goes to the lower index.  w[t,i] is the softmax over all E logits
 * renormalised over the selection (equal to the softmax over the k selected
 * logits) and sums to 1.  logits_out ([T,E] fp32) may be NULL.
 *   router_w [E,H] fp32, x [T,H] fp32, idx [T,k] int32, w [T,k] fp32.
 *   H a multiple of 4, all pointers 16-byte aligned, 1 <= k <= min(E, 16),
 *   E <= 2048, H <= 8192 (FMOE_ERR_UNSUPPORTED beyond).  T == 0 is a no-op.
 *   ws: fmoe_route_workspace_size(T, E) bytes. */
fmoe_status fmoe_route_topk(const float *router_w, const float *x, int32_t T, int32_t H,
                            int32_t E, int32_t k, int32_t *idx, float *w, float *logits_out,
                            void *ws, size_t ws_bytes, void *stream);
size_t fmoe_route_workspace_size(int32_t T, int32_t E);

/* y[n] = sum_k (code[n,k] * scale[n,k/G] + bias[n,k/G]) * x[k]  for one
 * quantised matrix ([WAS] "3. Handoptimierte Metal Compute-Shader": 4-bit /
 * 2-bit tiled matrix-vector multiply).  x [W->k] fp32, y [W->n] fp32, both
 * 16-byte aligned; y must not overlap x.  No workspace. */
fmoe_status fmoe_dequant_gemv(const fmoe_qmat *W, const fmoe_qformat *fmt, const float *x,
                              float *y, void *stream);

/* One expert FFN on one token: y = deq(down) (silu(deq(gate) x) * deq(up) x),
 * silu(z) = z / (1 + exp(-z)) ([WAS] section 3: fused SwiGLU).  gate/up must be
 * [I x H], down [H x I].  x [H], y [H] fp32, 16-byte aligned, not overlapping.
 *   ws: fmoe_expert_ffn_workspace_size(e, fmt) bytes. */
fmoe_status fmoe_expert_ffn(const fmoe_expert *e, const fmoe_qformat *fmt, const float *x,
                            float *y, void *ws, size_t ws_bytes, void *stream);
size_t fmoe_expert_ffn_workspace_size(const fmoe_expert *e, const fmoe_qformat *fmt);

/* The whole MoE layer for T tokens:
 *   route (as fmoe_route_topk) -> for each token, the k routed experts and the
 *   shared expert (slab E) run as in fmoe_expert_ffn ->
 *   moe[t]  = sum_i w[t,i] * FFN_{idx[t,i]}(x[t]) + g[t] * FFN_shared(x[t]),
 *             g[t] = sigmoid(shared_gate_w . x[t])
 *   h_out[t] = residual[t] + moe[t]                     (the new residual)
 *   y_out[t] = norm_w * h / sqrt(mean(h^2) + norm_eps)   (input of the next layer)
 * Indices never leave the device, so layers chain by passing y_out and h_out
 * of one call as x and residual of the next.
 *   x, residual, h_out, y_out: [T,H] fp32.  residual may alias x and h_out may
 *   alias residual; no other overlap.  idx_out [T,k] int32, w_out [T,k] fp32
 *   and moe_out [T,H] fp32 (before the residual) may each be NULL.
 *   ws: fmoe_workspace_size(L, T) bytes.  T == 0 is a no-op. */
fmoe_status fmoe_moe_layer_forward(const fmoe_layer *L, int32_t T, const float *x,
                                   const float *residual, float *h_out, float *y_out,
                                   int32_t *idx_out, float *w_out, float *moe_out,
                                   void *ws, size_t ws_bytes, void *stream);
size_t fmoe_workspace_size(const fmoe_layer *L, int32_t T);

#ifdef __cplusplus
}
#endif

#endif /* FMOE_H */
